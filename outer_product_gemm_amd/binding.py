"""Python binding of liboutprod.so: argument marshalling only.

The names follow the C ABI in ``include/outprod.h``:

* :func:`out_prod` / :func:`out_prod_ex` take raw device addresses (ints), the
  ``ne``/``nb`` arrays and a ``hipStream_t`` address, exactly like the C calls;
* :func:`out_prod_plan` runs the host-side checks and reports the launch;
* :func:`out_prod_id_back` / :func:`out_prod_id_back_plan`: MUL_MAT_ID_BACK;
* :func:`out_prod_strerror` / :func:`out_prod_version`.

:func:`out_prod_tensors` is a convenience that reads ``ne``/``nb`` off torch
tensors and uses torch's current stream.  Every step of the computation runs
in the library's HIP kernels; if the library is missing, the first call raises.

torch is imported before the library is loaded: torch ships its own
``libamdhip64.so.7``, and loading it first makes the library bind to the same
HIP runtime (same SONAME), so torch's device pointers and streams are valid in
both.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (must precede loading the library; see above)

# a types (GGUF ids; include/outprod.h OUTPROD_TYPE_*)
F32, F16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0 = 0, 1, 2, 3, 6, 7, 8
Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, BF16 = 10, 11, 12, 13, 14, 30
BLOCK_VALUES = {F32: 1, F16: 1, BF16: 1, Q4_0: 32, Q4_1: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32,
                Q2_K: 256, Q3_K: 256, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {F32: 4, F16: 2, BF16: 2, Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, Q8_0: 34,
               Q2_K: 84, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210}

OUTPROD_OK = 0
STATUS = {
    -1: "E_NULL", -2: "E_TYPE", -3: "E_SHAPE", -4: "E_K", -5: "E_DST_SHAPE", -6: "E_BCAST",
    -7: "E_QK", -8: "E_LAYOUT", -9: "E_ALIAS", -10: "E_RANGE", -11: "E_KERNEL", -12: "E_HIP",
    -13: "E_CAPTURE", -14: "E_WORKSPACE", -15: "E_SCRATCH",
}
KERNEL_AUTO, KERNEL_SKINNY, KERNEL_TILED, KERNEL_ZERO, KERNEL_NONE = 0, 1, 2, 3, 4
KERNEL_NAMES = {1: "skinny", 2: "tiled", 3: "zero", 4: "none"}
# Configuration indices each family accepts when forced (out_prod_ex bits
# 8-15): the tiled OUT_PROD menu, the grouped MUL_MAT_ID_BACK kernel's tiles.
TILED_CONFIGS = tuple(range(15)) + (19, 20)
ID_CONFIGS = (0, 1, 2, 4, 8, 10, 11, 12, 13, 15, 16, 17, 18)


def kernel_code(family: int, config: int = None, splits: int = None, group_m: int = None) -> int:
    """out_prod_ex's kernel argument: a family, optionally with a forced
    configuration index (as reported by out_prod_plan's ``variant``), a
    forced split count of K (1 = no split) and a forced tile order of the
    tiled kernel: tiles walk groups of ``group_m`` (1-127) tiles along i0 (as
    reported by out_prod_plan's ``group_m``)."""
    code = family | ((config + 1) << 8 if config is not None else 0)
    code |= splits << 16 if splits is not None else 0
    return code | (group_m << 24 if group_m is not None else 0)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboutprod.so")
# The library ABI this binding's structures and signatures match.
ABI_VERSION = 3

# Every symbol the header declares.
EXPORTS = ("out_prod", "out_prod_ex", "out_prod_plan", "out_prod_id_back", "out_prod_id_back_ex",
           "out_prod_id_back_plan", "out_prod_noalloc", "out_prod_release_stream", "out_prod_workspace_count",
           "out_prod_strerror", "out_prod_version")
_I64x16 = ctypes.c_int64 * 16


class OutProdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("out_prod failed: %s (%d): %s" % (STATUS.get(status, "?"), status, message))
        self.status = status


class outprod_plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("tile_k", ctypes.c_int), ("block", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("grid", ctypes.c_int64), ("slices", ctypes.c_int64), ("dps2", ctypes.c_int64),
                ("dps3", ctypes.c_int64), ("flops", ctypes.c_int64), ("variant", ctypes.c_int),
                ("swapped", ctypes.c_int), ("splits", ctypes.c_int), ("ksplit", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("group_m", ctypes.c_int),
                ("reserved", ctypes.c_int)]


_I64x12 = ctypes.c_int64 * 12
_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load liboutprod.so (once per process; later calls return the loaded
    library whatever the path).  Raises if it has not been built or if its
    ABI version is not the one this binding was written for."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("liboutprod.so is not built (%s); run __graft_entry__.build() "
                                   "or python -m outer_product_gemm_amd.build" % path)
            lib = ctypes.CDLL(path)
            vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
            lib.out_prod.argtypes = [vp, ctypes.c_int, vp, vp, i64p, i64p, vp]
            lib.out_prod.restype = ctypes.c_int
            lib.out_prod_ex.argtypes = [vp, ctypes.c_int, vp, vp, i64p, i64p, vp, ctypes.c_int]
            lib.out_prod_ex.restype = ctypes.c_int
            lib.out_prod_plan.argtypes = [vp, ctypes.c_int, vp, vp, i64p, i64p, ctypes.c_int,
                                          ctypes.POINTER(outprod_plan)]
            lib.out_prod_plan.restype = ctypes.c_int
            lib.out_prod_id_back.argtypes = [vp, ctypes.c_int, vp, vp, vp, i64p, i64p, vp]
            lib.out_prod_id_back.restype = ctypes.c_int
            lib.out_prod_id_back_ex.argtypes = [vp, ctypes.c_int, vp, vp, vp, i64p, i64p, vp,
                                                ctypes.c_int]
            lib.out_prod_id_back_ex.restype = ctypes.c_int
            lib.out_prod_id_back_plan.argtypes = [vp, ctypes.c_int, vp, vp, vp, i64p, i64p,
                                                  ctypes.c_int, ctypes.POINTER(outprod_plan)]
            lib.out_prod_id_back_plan.restype = ctypes.c_int
            lib.out_prod_noalloc.argtypes = [vp, ctypes.c_int, vp, vp, i64p, i64p, vp]
            lib.out_prod_noalloc.restype = ctypes.c_int
            lib.out_prod_release_stream.argtypes = [vp]
            lib.out_prod_release_stream.restype = ctypes.c_int
            lib.out_prod_workspace_count.argtypes = [ctypes.POINTER(ctypes.c_int)]
            lib.out_prod_workspace_count.restype = ctypes.c_int
            lib.out_prod_strerror.argtypes = [ctypes.c_int]
            lib.out_prod_strerror.restype = ctypes.c_char_p
            lib.out_prod_version.restype = ctypes.c_int
            got = int(lib.out_prod_version())
            if got != ABI_VERSION:
                raise RuntimeError("%s has ABI version %d, this binding needs %d: rebuild it "
                                   "(__graft_entry__.build())" % (path, got, ABI_VERSION))
            _lib = lib
    return _lib


def _arr12(x):
    vals = [int(v) for v in x]
    if len(vals) != 12:
        raise ValueError("ne/nb must have 12 entries")
    return _I64x12(*vals)


def _arr16(x):
    vals = [int(v) for v in x]
    if len(vals) != 16:
        raise ValueError("ne/nb must have 16 entries")
    return _I64x16(*vals)


def _check(status: int) -> None:
    if status != OUTPROD_OK:
        raise OutProdError(status, out_prod_strerror(status))


def out_prod_release_stream(stream: int = 0) -> None:
    """C ``out_prod_release_stream``: wait for ``stream`` and free the
    workspace the library holds for it."""
    _check(load_library().out_prod_release_stream(stream or None))


def out_prod_workspace_count() -> int:
    """C ``out_prod_workspace_count``: workspaces held on the current device."""
    n = ctypes.c_int(0)
    _check(load_library().out_prod_workspace_count(ctypes.byref(n)))
    return n.value


def out_prod_strerror(status: int) -> str:
    return load_library().out_prod_strerror(int(status)).decode()


def out_prod_version() -> int:
    return int(load_library().out_prod_version())


def out_prod(a: int, a_type: int, b: int, dst: int, ne, nb, stream: int = 0) -> None:
    """C ``out_prod`` on raw device addresses.  Raises OutProdError on a nonzero status."""
    _check(load_library().out_prod(a or None, int(a_type), b or None, dst or None,
                                   _arr12(ne), _arr12(nb), stream or None))


def out_prod_ex(a: int, a_type: int, b: int, dst: int, ne, nb, stream: int = 0,
                kernel: int = KERNEL_AUTO) -> None:
    """C ``out_prod_ex``: out_prod with the kernel family forced."""
    _check(load_library().out_prod_ex(a or None, int(a_type), b or None, dst or None,
                                      _arr12(ne), _arr12(nb), stream or None, int(kernel)))


def out_prod_noalloc(a: int, a_type: int, b: int, dst: int, ne, nb, stream: int = 0) -> None:
    """C ``out_prod_noalloc``: out_prod that allocates nothing (split partials
    in the library's static device scratch).  Raises OutProdError on a
    nonzero status."""
    _check(load_library().out_prod_noalloc(a or None, int(a_type), b or None, dst or None,
                                           _arr12(ne), _arr12(nb), stream or None))


def out_prod_noalloc_status(a: int, a_type: int, b: int, dst: int, ne, nb, stream: int = 0) -> int:
    """``out_prod_noalloc`` returning the raw status instead of raising."""
    return int(load_library().out_prod_noalloc(a or None, int(a_type), b or None, dst or None,
                                               _arr12(ne), _arr12(nb), stream or None))


def out_prod_status(a: int, a_type: int, b: int, dst: int, ne, nb, stream: int = 0,
                    kernel: int = KERNEL_AUTO) -> int:
    """``out_prod_ex`` returning the raw status instead of raising."""
    return int(load_library().out_prod_ex(a or None, int(a_type), b or None, dst or None,
                                          _arr12(ne), _arr12(nb), stream or None, int(kernel)))


def out_prod_plan(a: int, a_type: int, b: int, dst: int, ne, nb, kernel: int = KERNEL_AUTO) -> dict:
    """C ``out_prod_plan``: host-side checks and the launch a call would make."""
    p = outprod_plan()
    _check(load_library().out_prod_plan(a or None, int(a_type), b or None, dst or None,
                                        _arr12(ne), _arr12(nb), int(kernel), ctypes.byref(p)))
    d = {name: getattr(p, name) for name, _ in outprod_plan._fields_}
    d["kernel_name"] = KERNEL_NAMES.get(d["kernel"], "?")
    return d


def out_prod_id_back(as_: int, as_type: int, g: int, ids: int, dst: int, ne, nb,
                     stream: int = 0) -> None:
    """C ``out_prod_id_back`` (MUL_MAT_ID_BACK) on raw device addresses; ne/nb have
    16 entries (as, g, ids, dst).  Raises OutProdError on a non-zero status."""
    _check(load_library().out_prod_id_back(as_ or None, int(as_type), g or None, ids or None,
                                           dst or None, _arr16(ne), _arr16(nb), stream or None))


def out_prod_id_back_status(as_: int, as_type: int, g: int, ids: int, dst: int, ne, nb,
                            stream: int = 0, kernel: int = KERNEL_AUTO) -> int:
    """``out_prod_id_back_ex`` returning the raw status instead of raising."""
    return int(load_library().out_prod_id_back_ex(as_ or None, int(as_type), g or None, ids or None,
                                                  dst or None, _arr16(ne), _arr16(nb),
                                                  stream or None, int(kernel)))


def out_prod_id_back_plan(as_: int, as_type: int, g: int, ids: int, dst: int, ne, nb,
                          kernel: int = KERNEL_AUTO) -> dict:
    """C ``out_prod_id_back_plan``: host-side checks and the launch a call would make."""
    p = outprod_plan()
    _check(load_library().out_prod_id_back_plan(as_ or None, int(as_type), g or None, ids or None,
                                                dst or None, _arr16(ne), _arr16(nb), int(kernel),
                                                ctypes.byref(p)))
    d = {name: getattr(p, name) for name, _ in outprod_plan._fields_}
    d["kernel_name"] = KERNEL_NAMES.get(d["kernel"], "?")
    return d


def id_back_plan_status(as_: int, as_type: int, g: int, ids: int, dst: int, ne, nb,
                        kernel: int = KERNEL_AUTO) -> int:
    """``out_prod_id_back_plan`` returning the raw status instead of raising."""
    p = outprod_plan()
    return int(load_library().out_prod_id_back_plan(as_ or None, int(as_type), g or None,
                                                    ids or None, dst or None, _arr16(ne), _arr16(nb),
                                                    int(kernel), ctypes.byref(p)))


def plan_status(a: int, a_type: int, b: int, dst: int, ne, nb, kernel: int = KERNEL_AUTO) -> int:
    """``out_prod_plan`` returning the raw status instead of raising."""
    p = outprod_plan()
    return int(load_library().out_prod_plan(a or None, int(a_type), b or None, dst or None,
                                            _arr12(ne), _arr12(nb), int(kernel), ctypes.byref(p)))


# ---------------------------------------------------------------- torch tensors

# dtypes an f32 / f16 / bf16 ``a`` may have (2-byte integer tensors may hold
# the bits of the half types); block-quantized ``a`` is uint8
_A_DTYPES = {F32: (torch.float32,), F16: (torch.float16, torch.int16),
             BF16: (torch.bfloat16, torch.int16)}


def tensor_ne_nb(a: torch.Tensor, a_type: int, b: torch.Tensor, out: torch.Tensor, a_ne0=None):
    """ggml ne/nb of torch tensors laid out (ne3, ne2, ne1, ne0) (fewer dims are
    padded with leading 1s).  An f32 / f16 / bf16 ``a`` is a tensor of that
    dtype (or of 2-byte integers holding the bits); a block-quantized ``a`` is
    a uint8 tensor whose last dim is the row's bytes; ``a_ne0`` gives its
    value count.  b and out must be float32.  Raises ValueError for any other
    dtype (byte strides are the element strides times the element size, so
    a wrong dtype would describe memory the tensor does not own)."""
    if a_type not in BLOCK_VALUES:
        raise ValueError("unknown a_type %r" % (a_type,))
    want = _A_DTYPES.get(a_type, (torch.uint8,))
    if a.dtype not in want:
        raise ValueError("a has dtype %s; a_type %d needs %s" % (a.dtype, a_type, " or ".join(map(str, want))))
    if b.dtype != torch.float32:
        raise ValueError("b must be float32, not %s" % b.dtype)
    if out.dtype != torch.float32:
        raise ValueError("out must be float32, not %s" % out.dtype)
    for name, t in (("a", a), ("b", b), ("out", out)):
        if t.dim() > 4:
            raise ValueError("%s has %d dims; at most 4" % (name, t.dim()))

    def four(t):
        shape = [1] * (4 - t.dim()) + list(t.shape)
        stride = [0] * (4 - t.dim()) + list(t.stride())
        return shape[::-1], [t.element_size() * x for x in stride[::-1]]
    ash, ast = four(a)
    bsh, bst = four(b)
    osh, ost = four(out)
    if BLOCK_VALUES[a_type] == 1:
        a_ne, a_nb = ash, ast
    else:
        if a_ne0 is None:
            a_ne0 = ash[0] // BLOCK_BYTES[a_type] * BLOCK_VALUES[a_type]
        a_ne = [a_ne0] + ash[1:]
        a_nb = [BLOCK_BYTES[a_type]] + list(ast[1:])
    return a_ne + bsh + osh, a_nb + bst + ost


def out_prod_tensors(a: torch.Tensor, a_type: int, b: torch.Tensor, out: torch.Tensor = None,
                     a_ne0: int = None, kernel: int = KERNEL_AUTO, stream=None) -> torch.Tensor:
    """OUT_PROD of torch device tensors on the current (or given) stream.

    a: f32 / f16 / bf16 (ne03, ne02, K, ne00), or uint8 (ne03, ne02, K, row_bytes)
       for the block types;
    b: f32 (ne13, ne12, K, ne10); out: f32 (ne13, ne12, ne10, ne00), allocated if None.
    All three must be on the same GPU (ValueError otherwise, before any launch).
    """
    if b.device.type != "cuda":
        raise ValueError("b must be a GPU tensor, not on %s" % b.device)
    if out is None:
        bsh = [1] * (4 - b.dim()) + list(b.shape)
        if BLOCK_VALUES.get(a_type) == 1:
            ne00 = a.shape[-1]
        elif a_type in BLOCK_VALUES:
            ne00 = a_ne0 if a_ne0 is not None else a.shape[-1] // BLOCK_BYTES[a_type] * BLOCK_VALUES[a_type]
        else:
            raise ValueError("unknown a_type %r" % (a_type,))
        out = torch.empty((bsh[0], bsh[1], bsh[3], ne00), dtype=torch.float32, device=b.device)
    for name, t in (("a", a), ("out", out)):
        if t.device != b.device:
            raise ValueError("%s is on %s, b on %s: all tensors must be on one GPU" % (name, t.device, b.device))
    ne, nb = tensor_ne_nb(a, a_type, b, out, a_ne0)
    if stream is None:
        stream = torch.cuda.current_stream(b.device)
    out_prod_ex(a.data_ptr(), a_type, b.data_ptr(), out.data_ptr(), ne, nb, stream.cuda_stream, kernel)
    return out
