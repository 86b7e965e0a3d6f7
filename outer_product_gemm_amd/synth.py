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

# GGUF type ids of the a (src0) storage types
F32, F16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0 = 0, 1, 2, 3, 6, 7, 8
Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, BF16 = 10, 11, 12, 13, 14, 30
TYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", Q4_0: "q4_0", Q4_1: "q4_1", Q5_0: "q5_0",
              Q5_1: "q5_1", Q8_0: "q8_0", Q2_K: "q2_K", Q3_K: "q3_K", Q4_K: "q4_K",
              Q5_K: "q5_K", Q6_K: "q6_K"}
BLOCK_VALUES = {F32: 1, F16: 1, BF16: 1, Q4_0: 32, Q4_1: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32,
                Q2_K: 256, Q3_K: 256, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {F32: 4, F16: 2, BF16: 2, Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, Q8_0: 34,
               Q2_K: 84, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210}
QUANT_TYPES = (Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K)
# Byte offsets of a block's fp16 fields: (offset, role) with role "scale" (a
# positive multiplier, d or dmin) or "offset" (q4_1 / q5_1's additive m).
# Every other byte of a block (codes, packed sub-block scales, high bits) is
# drawn uniform, so each of those fields is uniform over its range.
HALF_FIELDS = {
    Q4_0: ((0, "scale"),), Q4_1: ((0, "scale"), (2, "offset")), Q5_0: ((0, "scale"),),
    Q5_1: ((0, "scale"), (2, "offset")), Q8_0: ((0, "scale"),),
    Q2_K: ((80, "scale"), (82, "scale")), Q3_K: ((108, "scale"),),
    Q4_K: ((0, "scale"), (2, "scale")), Q5_K: ((0, "scale"), (2, "scale")), Q6_K: ((208, "scale"),),
}


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


def block_rows(rng, a_type: int, nrows: int, ne00: int, d_range=(1e-3, 1e-2),
               m_range=(-0.1, 0.0), half_bits=None) -> np.ndarray:
    """(nrows, row_bytes) uint8 rows of any block type: uniform random bytes,
    then every fp16 field set to fp16(U(d_range)) (scales) or fp16(U(m_range))
    (q4_1 / q5_1 offsets); half_bits = {"scale": bits, "offset": bits} fixes
    those fields to one fp16 bit pattern instead."""
    nblk = ne00 // BLOCK_VALUES[a_type]
    bb = BLOCK_BYTES[a_type]
    out = rng.integers(0, 256, size=(nrows, nblk, bb), dtype=np.uint8)
    for off, role in HALF_FIELDS[a_type]:
        if half_bits is not None and role in half_bits:
            h = np.full((nrows, nblk), half_bits[role], dtype=np.uint16)
        else:
            lo, hi = d_range if role == "scale" else m_range
            h = fp16_bits(rng.uniform(lo, hi, size=(nrows, nblk)))
        out[:, :, off:off + 2] = h.reshape(nrows, nblk, 1).view(np.uint8).reshape(nrows, nblk, 2)
    return out.reshape(nrows, nblk * bb)


def quant_rows(rng, a_type: int, nrows: int, ne00: int, **kw) -> np.ndarray:
    if a_type == Q8_0:
        return q8_0_rows(rng, nrows, ne00, **kw)
    if a_type == Q4_K:
        return q4_K_rows(rng, nrows, ne00, **kw)
    if a_type in QUANT_TYPES:
        return block_rows(rng, a_type, nrows, ne00, **kw)
    raise ValueError("not a quantized type: %r" % a_type)


def half_rows(rng, a_type: int, shape, std: float = 1.0) -> np.ndarray:
    """uint16 f16 or bf16 patterns of N(0, std) values: f16 by numpy's
    round-to-nearest conversion, bf16 as the top half of the float32 bits."""
    x = normal_f32(rng, shape, std)
    if a_type == F16:
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Instance:
    """One OUT_PROD problem: host buffers plus the ggml ne/nb that address them."""
    name: str
    a_type: int
    a: np.ndarray          # f32 / uint16 (f16, bf16) (ne03, ne02, K, ne00), or uint8
                           # (ne03, ne02, K, row_bytes) for block types
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
    elif a_type in (F16, BF16):
        a = half_rows(rng, a_type, (ne03, ne02, K, ne00), a_std)
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
    # the pages' two smaller per-op q4_K training shapes (n = 1024)
    "q4_K_1536x1536": (Q4_K, (1536, 1536, 1, 1), (1024, 1536, 1, 1), 53, 1.0, "normal",
                       "q4_K weight x f32 gradient, m 1536 k 1536 n 1024"),
    "q4_K_5120x5120": (Q4_K, (5120, 5120, 1, 1), (1024, 5120, 1, 1), 54, 1.0, "normal",
                       "q4_K weight x f32 gradient, m 5120 k 5120 n 1024"),
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


# Every a type at the 27B up-projection shape (m 5120, k 17408, n 1024): the
# frozen-weight types out_prod reads (pages: the MUL_MAT_ID_BACK page's list,
# "out_prod's set").
TYPE_SWEEP = {}
for _t in (F32, F16, BF16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K):
    if _t == Q4_K:
        TYPE_SWEEP["q4_K_5120x17408"] = WORKLOADS["q4_K_5120x17408"]
        continue
    TYPE_SWEEP["%s_5120x17408" % TYPE_NAMES[_t]] = (
        _t, (5120, 17408, 1, 1), (1024, 17408, 1, 1), 80 + _t, 0.02 if _t in (F32, F16, BF16) else 1.0,
        "normal", "%s weight x f32 gradient, m 5120 k 17408 n 1024" % TYPE_NAMES[_t])
WORKLOADS.update(TYPE_SWEEP)
# ... and at the 27B down-projection's input-gradient shape (m 17408, k 5120,
# n 1024), the 272 x 128 tile with loader waves.
TYPE_SWEEP_DOWN = {}
for _t in (F32, F16, BF16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K):
    if _t == Q4_K:
        TYPE_SWEEP_DOWN["q4_K_17408x5120"] = WORKLOADS["q4_K_17408x5120"]
        continue
    TYPE_SWEEP_DOWN["%s_17408x5120" % TYPE_NAMES[_t]] = (
        _t, (17408, 5120, 1, 1), (1024, 5120, 1, 1), 120 + _t, 0.02 if _t in (F32, F16, BF16) else 1.0,
        "normal", "%s weight x f32 gradient, m 17408 k 5120 n 1024" % TYPE_NAMES[_t])
WORKLOADS.update(TYPE_SWEEP_DOWN)

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


# ---------------------------------------------------------------- MUL_MAT_ID_BACK inputs

@dataclass
class MoeInstance:
    """One MUL_MAT_ID_BACK problem: frozen experts, the output gradient of
    MUL_MAT_ID, the routing ids, and the ggml ne/nb[16] of (as, g, ids, dst)."""
    name: str
    a_type: int
    a: np.ndarray      # experts: f32/uint16 (n_expert, K, ne00) or uint8 (n_expert, K, row_bytes)
    g: np.ndarray      # f32 (n_tokens, n_used, K): g[t, i, r]
    ids: np.ndarray    # int32 (n_tokens, n_used)
    ne: list
    nb: list
    seed: int = 0
    note: str = ""

    @property
    def dst_shape(self):
        return (self.ne[14], self.ne[13], self.ne[12])


def moe_ne_nb(a_type: int, ne00: int, K: int, n_expert: int, n_used: int, n_tokens: int):
    """ne[16], nb[16] for contiguous experts, gradient, ids and dst."""
    rb = row_bytes(a_type, ne00)
    ne = [ne00, K, n_expert, 1, K, n_used, n_tokens, 1, n_used, n_tokens, 1, 1,
          ne00, n_used, n_tokens, 1]
    nb = [BLOCK_BYTES[a_type], rb, rb * K, rb * K * n_expert,
          4, 4 * K, 4 * K * n_used, 4 * K * n_used * n_tokens,
          4, 4 * n_used, 4 * n_used * n_tokens, 4 * n_used * n_tokens,
          4, 4 * ne00, 4 * ne00 * n_used, 4 * ne00 * n_used * n_tokens]
    return ne, nb


def top_k_ids(rng, n_expert: int, n_used: int, n_tokens: int) -> np.ndarray:
    """int32 (n_tokens, n_used): for each token, n_used distinct experts drawn
    uniformly (the indices of the n_used largest of n_expert uniform draws)."""
    u = rng.random((n_tokens, n_expert))
    return np.argsort(-u, axis=1)[:, :n_used].astype(np.int32)


def make_moe_instance(name: str, a_type: int, ne00: int, K: int, n_expert: int, n_used: int,
                      n_tokens: int, seed: int, a_std: float = 1.0, note: str = "") -> MoeInstance:
    """Draw the experts, then the routing, then g from PCG64(seed)."""
    rng = rng_for(seed)
    if a_type == F32:
        a = normal_f32(rng, (n_expert, K, ne00), a_std)
    elif a_type in (F16, BF16):
        a = half_rows(rng, a_type, (n_expert, K, ne00), a_std)
    else:
        a = quant_rows(rng, a_type, n_expert * K, ne00).reshape(n_expert, K, -1)
    ids = top_k_ids(rng, n_expert, n_used, n_tokens)
    g = normal_f32(rng, (n_tokens, n_used, K))
    ne, nb = moe_ne_nb(a_type, ne00, K, n_expert, n_used, n_tokens)
    return MoeInstance(name, a_type, a, g, ids, ne, nb, seed, note)


# name -> (a_type, ne00, K, n_expert, n_used, n_tokens, seed, note).  A
# mixture-of-experts FFN at the 4B's width (2560) with 64 q4_K experts of
# 1024 rows, 8 routed per token, 512 tokens: the up/gate projections'
# input gradient (ne00 = 2560, K = 1024) and the down projection's
# (ne00 = 1024, K = 2560).
MOE_WORKLOADS = {
    "moe_up_back_q4_K": (Q4_K, 2560, 1024, 64, 8, 512, 91,
                         "input gradient through 64 q4_K up-projection experts, 8 of 64 routed"),
    "moe_down_back_q4_K": (Q4_K, 1024, 2560, 64, 8, 512, 92,
                           "input gradient through 64 q4_K down-projection experts, 8 of 64 routed"),
}


def moe_workload(name: str) -> MoeInstance:
    a_type, ne00, K, ne_e, n_used, n_tok, seed, note = MOE_WORKLOADS[name]
    return make_moe_instance(name, a_type, ne00, K, ne_e, n_used, n_tok, seed, note=note)
