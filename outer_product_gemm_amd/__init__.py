"""OUT_PROD on MI355X (gfx950): hand-written HIP kernels behind a small C ABI.

    dst[i0,i1,i2,i3] = sum_k a[i0,k,i2/dps2,i3/dps3] * b[i1,k,i2,i3]

``a`` is f32, q8_0 or q4_K (dequantized in registers), ``b`` and ``dst`` are
f32, dps2 = ne12/ne02 and dps3 = ne13/ne03 (grouped-head broadcast).  Staging
and accumulation are fp32 throughout.

The compute path is ``liboutprod.so`` (C ABI declared in ``include/outprod.h``);
:mod:`outer_product_gemm_amd.binding` marshals arguments to it and nothing
else.  Importing this package does not load the library; the first call does,
and it raises if the library is missing.
"""
from .synth import F32, Q8_0, Q4_K  # noqa: F401

__all__ = ["F32", "Q8_0", "Q4_K", "binding"]


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(__name__ + ".binding")
    raise AttributeError(name)
