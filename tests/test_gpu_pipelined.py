"""Parity of the tiled kernel's full-tile loop with the CPU oracle.

A tiled workgroup whose tile lies wholly inside dst, with K a whole number of
stages and aligned operands, runs the pipelined loop (two raw register sets,
the decode spread over the MFMA steps, a wave-uniform tail round).  Its
prologue, steady state and tail take different branches for 1, 2, 3, 4 and
more stages, so every tiled configuration is forced here on shapes whose grid
holds full tiles next to ragged ones (i0 and i1), with K = 1..7 stages, for
every a type and both b layouts.  Gate as in test_gpu_parity: no NaN/Inf and
|gpu - ref| <= 1e-5 * sum_k |a||b| per element.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TOL = 1e-5
# stage rows (BK) of each tiled configuration, as out_prod_plan reports them
STAGE_ROWS = {0: 16, 1: 16, 2: 16, 3: 16, 4: 16, 5: 16, 6: 16,
              7: 32, 8: 32, 9: 32, 10: 32, 11: 32, 12: 16, 13: 16, 14: 32, 19: 32, 20: 32}
# i0 = 512 (a multiple of every block size): full 64/80/128/160/256-wide
# tiles and a ragged last one for 80, 160 and 272; i1 = 300: full
# 64/80/128/256-row tiles and a ragged last one
M, N = 512, 300
OTHER_TYPES = [synth.Q8_0, synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0,
               synth.Q5_1, synth.Q2_K, synth.Q3_K, synth.Q5_K, synth.Q6_K]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield


def _cases():
    """(a_type, stages, b slices over a slices, K-contiguous b)"""
    out = []
    for s in range(1, 8):
        out.append((synth.F32, s, 2 if s == 3 else 1, False))
        out.append((synth.Q4_K, s, 2 if s == 4 else 1, False))
        if s % 2:
            out.append((synth.F32, s, 1, True))
            out.append((synth.Q4_K, s, 1, True))
    for s in (5, 6):
        for t in OTHER_TYPES:
            out.append((t, s, 1, False))
    return out


def _stage_rows(inst, code):
    """BK of the forced configuration, from out_prod_plan on device buffers."""
    a_d = G.to_dev(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1))
    b_d = G.to_dev(inst.b)
    d_d = torch.empty(G.dst_extent_floats(inst.ne, inst.nb), dtype=torch.float32, device="cuda:0")
    return B.out_prod_plan(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), d_d.data_ptr(), inst.ne,
                           inst.nb, code)["tile_k"]


@pytest.mark.parametrize("cfg", B.TILED_CONFIGS)
def test_full_tiles_every_stage_count(cfg):
    code = B.kernel_code(B.KERNEL_TILED, cfg)
    bk = STAGE_ROWS[cfg]
    for a_type, stages, dps2, kt in _cases():
        K = bk * stages
        seed = zlib.crc32(repr(("pipe", cfg, a_type, stages, kt)).encode()) & 0x7FFFFFFF
        inst = synth.make_instance("pipe", a_type, (M, K, 1, 1), (N, K, dps2, 1), seed, b_kt=kt)
        if stages == 1 and a_type == synth.F32 and not kt:
            assert _stage_rows(inst, code) == bk
        G.log("case cfg", cfg, synth.TYPE_NAMES[a_type], "K", K, "stages", stages, "dps2", dps2,
              "b_kt", kt)
        gpu = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb, code)
        ref, den = oracle.out_prod(inst.a, inst.a_type, inst.b, inst.ne, inst.nb)
        res = oracle.check(gpu, ref, den, TOL)
        assert np.isfinite(gpu).all()
        assert res["ok"], (cfg, synth.TYPE_NAMES[a_type], K, kt, res)


@pytest.mark.parametrize("cfg", [8, 9, 14, 0, 4, 19])
def test_tile_order_every_way(cfg):
    """Tile orders forced through out_prod_ex and confirmed by the plan --
    i1 fastest (groups of 1), groups of 3 (a narrower last group when the
    tiles along i0 are not a multiple of 3), i0 fastest (127) -- on grids with
    broadcast slices, full and ragged tiles, for q4_K and f32 a."""
    for a_type, M, N, dps2 in ((synth.Q4_K, 4352, 256, 2), (synth.Q4_K, 512, 1100, 2),
                               (synth.F32, 4400, 130, 3), (synth.F32, 300, 900, 1),
                               (synth.Q4_K, 8192, 512, 2)):
        K = 64
        seed = zlib.crc32(repr(("order", cfg, a_type, M, N)).encode()) & 0x7FFFFFFF
        inst = synth.make_instance("order", a_type, (M, K, 1, 1), (N, K, dps2, 1), seed)
        a_d = G.to_dev(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1))
        b_d = G.to_dev(inst.b)
        d_d = torch.empty(G.dst_extent_floats(inst.ne, inst.nb), dtype=torch.float32, device="cuda:0")
        auto = B.out_prod_plan(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), d_d.data_ptr(), inst.ne,
                               inst.nb, B.kernel_code(B.KERNEL_TILED, cfg))
        tiles_m = -(-M // auto["tile_m"])
        assert 1 <= auto["group_m"] <= tiles_m
        ref, den = oracle.out_prod(inst.a, inst.a_type, inst.b, inst.ne, inst.nb)
        for g in (1, 3, 127):
            code = B.kernel_code(B.KERNEL_TILED, cfg, None, g)
            plan = B.out_prod_plan(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), d_d.data_ptr(), inst.ne,
                                   inst.nb, code)
            assert plan["group_m"] == min(g, tiles_m)
            G.log("case order cfg", cfg, synth.TYPE_NAMES[a_type], M, N, dps2, "group_m",
                  plan["group_m"], "tiles_m", tiles_m, "auto", auto["group_m"])
            gpu = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb, code)
            res = oracle.check(gpu, ref, den, TOL)
            assert np.isfinite(gpu).all()
            assert res["ok"], (cfg, synth.TYPE_NAMES[a_type], M, N, g, res)
