"""Helpers for the GPU tests: move seeded host inputs to the device, call the
library through its C ABI (raw addresses + ne/nb), and bring dst back."""
import sys

import numpy as np
import torch

from outer_product_gemm_amd import binding as B


def log(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def dst_extent_floats(ne, nb):
    ext = 4 * ne[8]
    for d in (1, 2, 3):
        if ne[8 + d] > 1:
            ext += (ne[8 + d] - 1) * nb[8 + d]
    return (ext + 3) // 4


def to_dev_at(x: np.ndarray, off: int):
    """Copy x's bytes to a fresh device buffer starting `off` bytes past a
    256-byte-aligned allocation; returns (buffer, address of x's first byte)."""
    raw = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    buf = torch.zeros(raw.size + off + 16, dtype=torch.uint8, device="cuda:0")
    buf[off:off + raw.size] = torch.from_numpy(raw).to("cuda:0")
    return buf, buf.data_ptr() + off


def run(a_host, a_type, b_host, ne, nb, kernel=0, sentinel=None, a_off=0, b_off=0):
    """OUT_PROD on cuda:0 via out_prod_ex.  a_host / b_host are host buffers
    that ne/nb address from their first byte; on the device they start a_off /
    b_off bytes past an aligned allocation.  Returns dst as a dense float32
    array (ne13, ne12, ne10, ne00) gathered through dst's strides."""
    keep = []
    a_ptr = b_ptr = 0
    if a_host is not None and a_host.size:
        buf, a_ptr = to_dev_at(a_host, a_off)
        keep.append(buf)
    if b_host is not None and b_host.size:
        buf, b_ptr = to_dev_at(b_host, b_off)
        keep.append(buf)
    n = max(1, dst_extent_floats(ne, nb))
    out = torch.full((n,), np.nan if sentinel is None else sentinel, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    B.out_prod_ex(a_ptr, a_type, b_ptr, out.data_ptr(), ne, nb, stream, kernel)
    torch.cuda.synchronize()
    flat = out.cpu().numpy()
    return gather(flat, ne, nb)


def gather(flat, ne, nb):
    ne00, ne10, ne12, ne13 = ne[8], ne[9], ne[10], ne[11]
    res = np.empty((ne13, ne12, ne10, ne00), dtype=np.float32)
    for i3 in range(ne13):
        for i2 in range(ne12):
            base = (i3 * nb[11] + i2 * nb[10]) // 4
            rows = base + (np.arange(ne10) * nb[9] // 4)[:, None] + np.arange(ne00)[None, :]
            res[i3, i2] = flat[rows]
    return res
