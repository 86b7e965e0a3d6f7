"""Operands and outputs past 4 GiB: every byte offset the kernels form must be
64-bit.  Inputs are drawn on the device from a seeded torch generator (a host
copy of several GiB would only slow the test); the oracle checks sampled dst
rows i1 through the sub-problem that keeps only those columns of b (each dst
row depends on its own column of b alone).  Gate as everywhere:
|gpu - ref| <= 1e-5 * sum_k |a||b|, no NaN/Inf.
"""
import numpy as np
import pytest
import torch

import oracle
from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TOL = 1e-5
GiB4 = 1 << 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield
    torch.cuda.empty_cache()


def device_normal(shape, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32)


def check_rows(a_host, a_type, a_ne, b_cols, rows, got):
    """b_cols: (K, n) host array, column c of b for dst row rows[c]; got:
    (n, ne00) GPU dst rows."""
    K = a_ne[1]
    ne, nb = synth.make_ne_nb(a_type, a_ne, (len(rows), K, 1, 1))
    ref, den = oracle.out_prod(a_host, a_type, np.ascontiguousarray(b_cols), ne, nb)
    res = oracle.check(got.reshape(1, 1, len(rows), -1), ref, den, TOL)
    G.log("   ", res)
    assert res["ok"], res
    assert np.isfinite(got).all()


def sample_rows(n, seed, k=24):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, 1, n - 2, n - 1] + list(rng.integers(0, n, k)))), dtype=np.int64)


def test_column_kernel_b_past_4GiB():
    """Rank-8 f32 a over a row-major b of 4.6 GB (column kernel)."""
    K, N = 1100, (1 << 20) + 48
    inst = synth.make_instance("big_col", synth.F32, (8, K, 1, 1), (16, K, 1, 1), 501)
    ne, nb = synth.make_ne_nb(synth.F32, (8, K, 1, 1), (N, K, 1, 1))
    assert K * N * 4 > GiB4
    p = B.out_prod_plan(0x10000000, synth.F32, 0x40000000000, 0x80000000000, ne, nb)
    G.log("case big_col b", K, "x", N, "plan", p["kernel_name"], p["tile_n"], p["grid"])
    assert p["kernel_name"] == "skinny"
    b = device_normal((K, N), 502)
    a = G.to_dev(inst.a)
    dst = torch.full((N, 8), float("nan"), dtype=torch.float32, device="cuda:0")
    B.out_prod(a.data_ptr(), synth.F32, b.data_ptr(), dst.data_ptr(), ne, nb,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = sample_rows(N, 503)
    idx = torch.from_numpy(rows).to("cuda:0")
    got = dst[idx].cpu().numpy()
    b_cols = b[:, idx].cpu().numpy()
    assert torch.isfinite(dst).all().item()
    del b, dst
    check_rows(inst.a, synth.F32, (8, K, 1, 1), b_cols, rows, got)


def test_tiled_kernel_q4K_b_past_4GiB():
    """q4_K a (in-register dequant) over a row-major b of 4.8 GB (tiled kernel)."""
    K, N, M = 4608, 262144, 256
    inst = synth.make_instance("big_q4K", synth.Q4_K, (M, K, 1, 1), (16, K, 1, 1), 511)
    ne, nb = synth.make_ne_nb(synth.Q4_K, (M, K, 1, 1), (N, K, 1, 1))
    assert K * N * 4 > GiB4
    p = B.out_prod_plan(0x10000000, synth.Q4_K, 0x40000000000, 0x80000000000, ne, nb)
    G.log("case big_q4K b", K, "x", N, "plan", p["kernel_name"], p["tile_m"], p["tile_n"], p["grid"])
    assert p["kernel_name"] == "tiled"
    b = device_normal((K, N), 512)
    a = G.to_dev(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1))
    dst = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda:0")
    B.out_prod(a.data_ptr(), synth.Q4_K, b.data_ptr(), dst.data_ptr(), ne, nb,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = sample_rows(N, 513)
    idx = torch.from_numpy(rows).to("cuda:0")
    got = dst[idx].cpu().numpy()
    b_cols = b[:, idx].cpu().numpy()
    assert torch.isfinite(dst).all().item()
    del b, dst
    check_rows(inst.a, synth.Q4_K, (M, K, 1, 1), b_cols, rows, got)


def test_tiled_kernel_dst_past_4GiB():
    """A dst of 4.6 GB (f32, short K, tiled kernel): stores past 4 GiB."""
    K, N, M = 4, 140000, 8192
    inst = synth.make_instance("big_dst", synth.F32, (M, K, 1, 1), (N, K, 1, 1), 521)
    assert M * N * 4 > GiB4
    p = B.out_prod_plan(0x10000000, synth.F32, 0x40000000000, 0x80000000000, inst.ne, inst.nb)
    G.log("case big_dst", M, "x", N, "plan", p["kernel_name"], p["tile_m"], p["tile_n"], p["grid"])
    assert p["kernel_name"] == "tiled"
    a = G.to_dev(inst.a)
    b = G.to_dev(inst.b)
    dst = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda:0")
    B.out_prod(a.data_ptr(), synth.F32, b.data_ptr(), dst.data_ptr(), inst.ne, inst.nb,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = sample_rows(N, 523)
    got = dst[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    assert torch.isfinite(dst).all().item()
    del dst
    b_cols = inst.b.reshape(K, N)[:, rows]
    check_rows(inst.a, synth.F32, (M, K, 1, 1), b_cols, rows, got)
