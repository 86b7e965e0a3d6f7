"""Parity with forced kernel configurations on seeded random shapes: every
tiled configuration (with and without split K, whole tiles and ragged ones,
short K of one to three stages), every column configuration, and every
grouped MUL_MAT_ID_BACK configuration, against the oracle.  The automatic
planner reaches only some configurations on the other tests' shapes; this
runs the rest through the same parity gate.  Cases are drawn once from a
fixed seed, so a failure names its case."""
import numpy as np
import pytest
import torch

import oracle
from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth
from tests import gpu_util as G
from tests.test_gpu_id_back import run_id

pytestmark = pytest.mark.gpu

TOL = 1e-5
TYPES = [synth.F32, synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0, synth.Q5_1,
         synth.Q8_0, synth.Q2_K, synth.Q3_K, synth.Q4_K, synth.Q5_K, synth.Q6_K]
# tiled configuration -> (tile height along i0, tile width along i1, stage rows)
TILED = {0: (128, 128, 16), 1: (160, 128, 16), 2: (160, 64, 16), 3: (272, 128, 16), 4: (64, 64, 16),
         5: (272, 64, 16), 6: (256, 128, 16), 7: (128, 128, 32), 8: (160, 128, 32), 9: (272, 128, 32),
         10: (160, 64, 32), 11: (64, 64, 32), 12: (128, 80, 16), 13: (64, 80, 16), 14: (80, 256, 32),
         19: (272, 128, 32), 20: (272, 128, 32)}
ID_CFGS = list(B.ID_CONFIGS)
assert sorted(TILED) == sorted(B.TILED_CONFIGS)
COLUMN_CFGS = 13


def _cases():
    rng = np.random.default_rng(20261204)
    out = []
    for cfg, (bm, bn, bk) in TILED.items():
        for j in range(4):
            a_type = int(rng.choice(TYPES))
            qk = synth.BLOCK_VALUES[a_type]
            if j % 2 == 0:   # whole tiles, whole stages; j == 0: one to three stages
                m, n = bm * int(rng.integers(1, 3)), bn * int(rng.integers(1, 3))
                K = bk * (int(rng.integers(1, 4)) if j == 0 else int(rng.integers(4, 12)))
            else:
                m, n, K = int(rng.integers(1, 2 * bm)), int(rng.integers(1, 2 * bn)), int(rng.integers(1, 400))
            if qk > 1:
                m = max(qk, (m + qk - 1) // qk * qk)
            splits = int(rng.choice([0, 2, 3])) if K >= 64 and j >= 2 else 0
            out.append(("tiled", a_type, m, n, K, int(rng.integers(1, 3)), bool(rng.integers(0, 2)), cfg,
                        splits, int(rng.integers(0, 2 ** 31 - 1))))
    for cfg in range(COLUMN_CFGS):
        for j in range(2):
            m = int(rng.choice([4, 8, 16, 24, 32, int(rng.integers(1, 40))]))
            n, K = int(rng.integers(1, 1200)), int(rng.integers(1, 1100))
            splits = int(rng.choice([0, 2, 4])) if K >= 256 else 0
            out.append(("column", synth.F32, m, n, K, int(rng.integers(1, 3)), bool(rng.integers(0, 2)), cfg,
                        splits, int(rng.integers(0, 2 ** 31 - 1))))
    # the loader-wave tiles (19, 20): every a type, K from one row to a few
    # stages (and its ring of three LDS stages wrapping several times),
    # ragged tiles in both directions, broadcast slices, splits
    for cfg in (19, 20):
        for a_type in TYPES:
            qk = synth.BLOCK_VALUES[a_type]
            m = int(rng.integers(1, 600))
            m = max(qk, (m + qk - 1) // qk * qk) if qk > 1 else m
            n = int(rng.integers(1, 300))
            K = int(rng.choice([1, 31, 32, 64, 96, 100, 224, int(rng.integers(1, 700))]))
            splits = int(rng.choice([0, 2, 3])) if K >= 64 else 0
            out.append(("tiled", a_type, m, n, K, int(rng.integers(1, 3)), bool(rng.integers(0, 2)), cfg,
                        splits, int(rng.integers(0, 2 ** 31 - 1))))
    for cfg in ID_CFGS:
        a_type = int(rng.choice(TYPES))
        qk = synth.BLOCK_VALUES[a_type]
        ne00 = qk * int(rng.integers(1, 5)) if qk > 1 else int(rng.integers(1, 300))
        K = int(rng.choice([16, 32, 96, 160, int(rng.integers(1, 300))]))
        E = int(rng.integers(1, 20))
        out.append(("id", a_type, ne00, K, E, int(rng.integers(1, min(E, 6) + 1)), int(rng.integers(1, 200)),
                    cfg, 0, int(rng.integers(0, 2 ** 31 - 1))))
    return out


CASES = _cases()


def _name(c):
    if c[0] == "id":
        return "id-cfg%d-%s-%dx%d-E%d" % (c[7], synth.TYPE_NAMES[c[1]], c[2], c[3], c[4])
    return "%s-cfg%d-x%d-%s-%dx%dx%d" % (c[0], c[7], c[8], synth.TYPE_NAMES[c[1]], c[2], c[3], c[4])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield


@pytest.mark.parametrize("case", CASES, ids=_name)
def test_forced_configuration(case):
    kind, a_type, p0, p1, p2, p3, p4, cfg, splits, seed = case
    if kind == "id":
        inst = synth.make_moe_instance("fz", a_type, p0, p1, p2, p3, p4, seed)
        G.log("case", _name(case), "seed", seed)
        gpu, _ = run_id(inst, kernel=B.kernel_code(B.KERNEL_TILED, cfg))
        ref, den = oracle.mul_mat_id_back(inst.a, inst.a_type, inst.g, inst.ids, inst.ne, inst.nb)
        res = oracle.check(gpu.reshape(ref.shape), ref, den, TOL)
        assert res["ok"], (case, res)
        return
    m, n, K, d2, kt = p0, p1, p2, p3, p4
    family = B.KERNEL_TILED if kind == "tiled" else B.KERNEL_SKINNY
    code = B.kernel_code(family, cfg, splits if splits else None)
    inst = synth.make_instance("fz", a_type, (m, K, 1, 1), (n, K, d2, 1), seed, b_kt=kt)
    st = B.plan_status(0x10000000, a_type, 0x40000000000, 0x80000000000, inst.ne, inst.nb, code)
    if B.STATUS.get(st) == "E_KERNEL":
        pytest.skip("the configuration refuses this layout (K-contiguous b in wide strips)")
    assert st == 0, B.STATUS.get(st)
    G.log("case", _name(case), "d2", d2, "kt" if kt else "rows", "seed", seed)
    gpu = G.run(inst.a, a_type, inst.b, inst.ne, inst.nb, kernel=code)
    ref, den = oracle.out_prod(inst.a, a_type, inst.b, inst.ne, inst.nb)
    res = oracle.check(gpu, ref, den, TOL)
    assert res["ok"], (case, res)
