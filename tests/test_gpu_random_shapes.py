"""Parity on random shapes: for every a type, seeded random cases with
any a width (f32/f16/bf16 1-40, block types 1-3 whole blocks), b widths 1-40,
K 1-300, slice broadcast factors 1-4 (dim 2) and 1-2 (dim 3) over 1-2 a
slices per dim, row-major or K-contiguous b, automatic kernel choice; and
medium cases (a 128-704 wide, b 64-600 wide, K up to 1024 and mostly a
whole number of 32-row stages) whose automatic plans run the tiled kernel's
full tiles, its pipelined loop and split K.  Each case is checked element by
element against the oracle with the parity gate.  The case lists are drawn
once from fixed seeds, so every run sees the same cases and a failure names
its case."""
import numpy as np
import pytest
import torch

import oracle
from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TOL = 1e-5
TYPES = [synth.F32, synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0, synth.Q5_1,
         synth.Q8_0, synth.Q2_K, synth.Q3_K, synth.Q4_K, synth.Q5_K, synth.Q6_K]
PER_TYPE = 8


def _cases():
    rng = np.random.default_rng(20261202)
    out = []
    for a_type in TYPES:
        qk = synth.BLOCK_VALUES[a_type]
        for _ in range(PER_TYPE):
            ne00 = int(rng.integers(1, 41)) if qk == 1 else qk * int(rng.integers(1, 4))
            ne10 = int(rng.integers(1, 41))
            K = int(rng.integers(1, 301))
            ne02, ne03 = int(rng.integers(1, 3)), int(rng.integers(1, 3))
            d2, d3 = int(rng.integers(1, 5)), int(rng.integers(1, 3))
            kt = bool(rng.integers(0, 2))
            seed = int(rng.integers(0, 2 ** 31 - 1))
            out.append((a_type, (ne00, K, ne02, ne03), (ne10, K, ne02 * d2, ne03 * d3), kt, seed))
    return out


CASES = _cases()


def _medium_cases():
    rng = np.random.default_rng(20261203)
    out = []
    for a_type in TYPES:
        qk = synth.BLOCK_VALUES[a_type]
        for _ in range(3):
            if qk == 1:
                ne00 = int(rng.integers(128, 705))
                if rng.integers(0, 2):
                    ne00 -= ne00 % 4  # 16-byte rows: the full-tile path
            else:
                ne00 = qk * int(rng.integers(max(1, 128 // qk), 704 // qk + 1))
            ne10 = int(rng.integers(64, 601))
            if rng.integers(0, 4):
                K = 32 * int(rng.integers(1, 33))  # whole stages
            else:
                K = int(rng.integers(1, 1025))
            ne02 = 1
            d2 = int(rng.integers(1, 3))
            kt = bool(rng.integers(0, 2))
            seed = int(rng.integers(0, 2 ** 31 - 1))
            out.append((a_type, (ne00, K, ne02, 1), (ne10, K, ne02 * d2, 1), kt, seed))
    return out


MEDIUM_CASES = _medium_cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-%s-%s" % (
    synth.TYPE_NAMES[c[0]], "x".join(map(str, c[1])), "x".join(map(str, c[2])), "kt" if c[3] else "rows"))
def test_random_small_shape(case):
    a_type, a_ne, b_ne, kt, seed = case
    inst = synth.make_instance("rand", a_type, a_ne, b_ne, seed, b_kt=kt)
    plan = B.out_prod_plan(0x10000000, a_type, 0x40000000000, 0x80000000000, inst.ne, inst.nb)
    G.log("case rand", synth.TYPE_NAMES[a_type], a_ne, b_ne, "kt" if kt else "rows", "seed", seed,
          plan["kernel_name"], plan["variant"], plan["splits"])
    gpu = G.run(inst.a, a_type, inst.b, inst.ne, inst.nb)
    ref, den = oracle.out_prod(inst.a, a_type, inst.b, inst.ne, inst.nb)
    res = oracle.check(gpu, ref, den, TOL)
    assert res["ok"], (case, res)
    assert np.isfinite(gpu).all()


@pytest.mark.parametrize("case", MEDIUM_CASES, ids=lambda c: "%s-%s-%s-%s" % (
    synth.TYPE_NAMES[c[0]], "x".join(map(str, c[1])), "x".join(map(str, c[2])), "kt" if c[3] else "rows"))
def test_random_medium_shape(case):
    test_random_small_shape(case)
