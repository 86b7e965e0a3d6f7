"""Seeded synthetic inputs for OUT_PROD.

This module is shared by the tests, the benchmark and the smoke check.  It holds
no arithmetic of the method: it only draws random numbers (numpy PCG64), packs
them into the storage formats and states the ggml ``ne``/``nb`` of each buffer.
Quantized blocks are drawn field by field: every bit of the packed scale/min
bytes and of the 4-bit codes is uniform, so each 6-bit scale, 6-bit min and
4-bit code is uniform over its range without the generator knowing the bit
positions.

Tensor conventions (ggml order, ne0 fastest):
  a   [ne00, K, ne02, ne03]  f32, or quantized rows of ne00 values
  b   [ne10, K, ne12, ne13]  f32
  dst [ne00, ne10, ne12, ne13] f32
As numpy arrays the shapes are reversed: a is (ne03, ne02, K, ne00) for f32 and
(ne03, ne02, K, row_bytes) uint8 for quantized types.

Workloads follow the pages' LoRA backward (rank 4/8/24 gradients at a 4B
model's shapes with 512-token ubatches, the 16-value-head over 4-key-head
delta-net backward, and q4_K weight x f32 gradient products with n = 1024 at
the 27B's 5120 / 17408 shapes).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32, Q8_0, Q4_K = 0, 8, 12
TYPE_NAMES = {F32: "f32", Q8_0: "q8_0", Q4_K: "q4_K"}
BLOCK_VALUES = {F32: 1, Q8_0: 32, Q4_K: 256}
BLOCK_BYTES = {F32: 4, Q8_0: 34, Q4_K: 144}


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def fp16_bits(values) -> np.ndarray:
    """IEEE binary16 bit patterns of float values (numpy's round-to-nearest conversion)."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def row_bytes(a_type: int, ne00: int) -> int:
    if ne00 % BLOCK_VALUES[a_type]:
        raise ValueError("width %d is not a multiple of the %s block" % (ne00, TYPE_NAMES[a_type]))
    return ne00 // BLOCK_VALUES[a_type] * BLOCK_BYTES[a_type]


def contiguous_nb(elem_bytes: int, row_nbytes: int, ne1: int, ne2: int) -> list:
    return [elem_bytes, row_nbytes, row_nbytes * ne1, row_nbytes * ne1 * ne2]


def make_ne_nb(a_type: int, a_ne, b_ne, b_kt: bool = False):
    """ne[12], nb[12] for contiguous a, b and dst of the given shapes.  With
    b_kt, b is stored K-contiguous: numpy shape (ne13, ne12, ne10, K), the
    transposed view a matmul backward passes for the input gradient."""
    ne00, K, ne02, ne03 = (int(x) for x in a_ne)
    ne10, K1, ne12, ne13 = (int(x) for x in b_ne)
    ne = [ne00, K, ne02, ne03, ne10, K1, ne12, ne13, ne00, ne10, ne12, ne13]
    nb_a = contiguous_nb(BLOCK_BYTES[a_type], row_bytes(a_type, ne00), K, ne02)
    if b_kt:
        nb_b = [4 * K1, 4, 4 * K1 * ne10, 4 * K1 * ne10 * ne12]
    else:
        nb_b = contiguous_nb(4, 4 * ne10, K1, ne12)
    nb_d = contiguous_nb(4, 4 * ne00, ne10, ne12)
    return ne, nb_a + nb_b + nb_d


def normal_f32(rng, shape, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(shape) * std).astype(np.float32)


def gradient_like_f32(rng, shape, scale: float = 1e3, frac: float = 0.005,
                      lo: float = 6.6e4, hi: float = 1.5e5) -> np.ndarray:
    """N(0,1)*scale with floor(frac*numel) entries replaced by +-U(lo, hi).

    The outliers stand for the training gradients the pages saw reach |x| of
    131273, past half precision's 65504."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    n = int(np.floor(frac * x.size))
    flat = x.reshape(-1)
    pos = rng.choice(x.size, size=n, replace=False)
    sign = np.where(rng.integers(0, 2, size=n) == 0, -1.0, 1.0)
    mag = rng.uniform(lo, hi, size=n)
    flat[pos] = (sign * mag).astype(np.float32)
    return x


def q8_0_rows(rng, nrows: int, ne00: int, d_range=(1e-3, 1e-2), d_bits=None,
              q_range=(-127, 127)) -> np.ndarray:
    """(nrows, row_bytes) uint8 q8_0 rows.  d = fp16(U(d_range)) unless d_bits
    (an fp16 bit pattern) is given; q uniform integers in q_range (inclusive)."""
    nblk = ne00 // 32
    out = np.empty((nrows, nblk, 34), dtype=np.uint8)
    if d_bits is None:
        d = fp16_bits(rng.uniform(d_range[0], d_range[1], size=(nrows, nblk)))
    else:
        d = np.full((nrows, nblk), d_bits, dtype=np.uint16)
    out[:, :, 0:2] = d.reshape(nrows, nblk, 1).view(np.uint8).reshape(nrows, nblk, 2)
    q = rng.integers(q_range[0], q_range[1] + 1, size=(nrows, nblk, 32)).astype(np.int8)
    out[:, :, 2:34] = q.view(np.uint8)
    return out.reshape(nrows, nblk * 34)


def q4_K_rows(rng, nrows: int, ne00: int, d_range=(1e-3, 1e-2), d_bits=None,
              dmin_bits=None) -> np.ndarray:
    """(nrows, row_bytes) uint8 q4_K rows.  d, dmin = fp16(U(d_range)) unless fixed
    bit patterns are given; the 12 packed scale/min bytes and the 128 code bytes
    are uniform random bytes."""
    nblk = ne00 // 256
    out = np.empty((nrows, nblk, 144), dtype=np.uint8)
    if d_bits is None:
        d = fp16_bits(rng.uniform(d_range[0], d_range[1], size=(nrows, nblk)))
    else:
        d = np.full((nrows, nblk), d_bits, dtype=np.uint16)
    if dmin_bits is None:
        dmin = fp16_bits(rng.uniform(d_range[0], d_range[1], size=(nrows, nblk)))
    else:
        dmin = np.full((nrows, nblk), dmin_bits, dtype=np.uint16)
    out[:, :, 0:2] = d.reshape(nrows, nblk, 1).view(np.uint8).reshape(nrows, nblk, 2)
    out[:, :, 2:4] = dmin.reshape(nrows, nblk, 1).view(np.uint8).reshape(nrows, nblk, 2)
    out[:, :, 4:144] = rng.integers(0, 256, size=(nrows, nblk, 140), dtype=np.uint8)
    return out.reshape(nrows, nblk * 144)


def quant_rows(rng, a_type: int, nrows: int, ne00: int, **kw) -> np.ndarray:
    if a_type == Q8_0:
        return q8_0_rows(rng, nrows, ne00, **kw)
    if a_type == Q4_K:
        return q4_K_rows(rng, nrows, ne00, **kw)
    raise ValueError("not a quantized type: %r" % a_type)


@dataclass
class Instance:
    """One OUT_PROD problem: host buffers plus the ggml ne/nb that address them."""
    name: str
    a_type: int
    a: np.ndarray          # f32 (ne03, ne02, K, ne00) or uint8 (ne03, ne02, K, row_bytes)
    b: np.ndarray          # f32 (ne13, ne12, K, ne10)
    ne: list
    nb: list
    seed: int = 0
    note: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def b_kt(self):
        return self.nb[5] == 4 and self.nb[4] != 4

    @property
    def dst_shape(self):
        ne = self.ne
        return (ne[11], ne[10], ne[9], ne[8])


def make_instance(name: str, a_type: int, a_ne, b_ne, seed: int, a_std: float = 1.0,
                  b_kind: str = "normal", note: str = "", b_kt: bool = False) -> Instance:
    """Draw a, then b (then b's outliers), from PCG64(seed).  b_kt stores the
    same b values K-contiguous (numpy shape (ne13, ne12, ne10, K))."""
    ne00, K, ne02, ne03 = (int(x) for x in a_ne)
    ne10, _, ne12, ne13 = (int(x) for x in b_ne)
    rng = rng_for(seed)
    if a_type == F32:
        a = normal_f32(rng, (ne03, ne02, K, ne00), a_std)
    else:
        a = quant_rows(rng, a_type, ne03 * ne02 * K, ne00).reshape(ne03, ne02, K, -1)
    if b_kind == "normal":
        b = normal_f32(rng, (ne13, ne12, K, ne10))
    elif b_kind == "gradient":
        b = gradient_like_f32(rng, (ne13, ne12, K, ne10))
    else:
        raise ValueError(b_kind)
    if b_kt:
        b = np.ascontiguousarray(b.transpose(0, 1, 3, 2))
    ne, nb = make_ne_nb(a_type, a_ne, b_ne, b_kt)
    return Instance(name, a_type, a, b, ne, nb, seed, note)


# name -> (a_type, a_ne, b_ne, seed, a_std, b_kind, note)
WORKLOADS = {
    "lora_r8_single": (F32, (8, 512, 1, 1), (2560, 512, 1, 1), 1, 1.0, "normal",
                       "LoRA rank-8 gradient, one slice, K = 512 tokens"),
    "deltanet_bcast": (F32, (128, 512, 4, 1), (128, 512, 16, 1), 2, 1.0, "gradient",
                       "grouped-head broadcast: 16 value heads over 4 key heads"),
    "lora_r4_2560": (F32, (4, 512, 1, 1), (2560, 512, 1, 1), 31, 0.02, "normal", "rank-4, 4B dim"),
    "lora_r4_9216": (F32, (4, 512, 1, 1), (9216, 512, 1, 1), 32, 0.02, "normal", "rank-4, 4B ffn"),
    "lora_r8_2560": (F32, (8, 512, 1, 1), (2560, 512, 1, 1), 33, 0.02, "normal", "rank-8, 4B dim"),
    "lora_r8_9216": (F32, (8, 512, 1, 1), (9216, 512, 1, 1), 34, 0.02, "normal", "rank-8, 4B ffn"),
    "lora_r24_2560": (F32, (24, 512, 1, 1), (2560, 512, 1, 1), 35, 0.02, "normal", "rank-24, 4B dim"),
    "lora_r24_9216": (F32, (24, 512, 1, 1), (9216, 512, 1, 1), 36, 0.02, "normal", "rank-24, 4B ffn"),
    "q8_0_5120": (Q8_0, (5120, 5120, 1, 1), (1024, 5120, 1, 1), 4, 1.0, "normal",
                  "frozen q8_0 weight x f32 gradient, 5120 x 5120, n = 1024"),
    "q4_K_5120x17408": (Q4_K, (5120, 17408, 1, 1), (1024, 17408, 1, 1), 51, 1.0, "normal",
                        "27B q4_K weight x f32 gradient, m 5120 k 17408 n 1024"),
    "q4_K_17408x5120": (Q4_K, (17408, 5120, 1, 1), (1024, 5120, 1, 1), 52, 1.0, "normal",
                        "27B q4_K weight x f32 gradient, m 17408 k 5120 n 1024"),
}


# The backward of one LoRA-adapted linear layer y = W x + B (A x) with W a
# frozen q4_K weight (in -> out), A [in -> r], B [r -> out], over T tokens.
# The matmul backward is entirely OUT_PROD (pages: "metal: OUT_PROD multiplies in
# float staging", body): the input gradient through a weight is
# out_prod(weight, grad^T) -- b is the transposed (K-contiguous) view of the
# gradient -- and a weight's gradient is out_prod(input, grad).
#   dx_W = out_prod(W, gy^T)   a: q4_K [in, out]   b: [T, out] K-contiguous
#   dB   = out_prod(h, gy)     a: [r, T]           b: [out, T]
#   dh   = out_prod(B, gy^T)   a: [r, out]         b: [T, out] K-contiguous
#   dA   = out_prod(x, dh)     a: [in, T]          b: [r, T]   (narrow b)
#   dx_A = out_prod(A, dh^T)   a: [in, r]          b: [T, r]   K-contiguous
def lora_linear_backward(prefix: str, n_in: int, n_out: int, rank: int, tokens: int, seed: int):
    return {
        prefix + "_dxW": (Q4_K, (n_in, n_out, 1, 1), (tokens, n_out, 1, 1), seed, 1.0, "normal",
                          "input gradient through the frozen q4_K weight", True),
        prefix + "_dB": (F32, (rank, tokens, 1, 1), (n_out, tokens, 1, 1), seed + 1, 0.02, "normal",
                         "LoRA B gradient", False),
        prefix + "_dh": (F32, (rank, n_out, 1, 1), (tokens, n_out, 1, 1), seed + 2, 0.02, "normal",
                         "gradient of the rank-r activation", True),
        prefix + "_dA": (F32, (n_in, tokens, 1, 1), (rank, tokens, 1, 1), seed + 3, 1.0, "normal",
                         "LoRA A gradient (narrow b)", False),
        prefix + "_dxA": (F32, (n_in, rank, 1, 1), (tokens, rank, 1, 1), seed + 4, 0.02, "normal",
                          "input gradient through A", True),
    }


LORA_BACKWARD = {
    "lora_4B_linear_backward": lora_linear_backward("lora4B", 2560, 9216, 8, 512, 61),
    "lora_27B_linear_backward": lora_linear_backward("lora27B", 5120, 17408, 8, 1024, 71),
}
for _group in LORA_BACKWARD.values():
    WORKLOADS.update(_group)


def workload(name: str, seed: int = None) -> Instance:
    spec = WORKLOADS[name]
    a_type, a_ne, b_ne, s, a_std, b_kind, note = spec[:7]
    b_kt = spec[7] if len(spec) > 7 else False
    return make_instance(name, a_type, a_ne, b_ne, s if seed is None else seed, a_std, b_kind, note,
                         b_kt=b_kt)
