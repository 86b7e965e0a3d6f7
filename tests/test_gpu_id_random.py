"""MUL_MAT_ID_BACK parity on seeded random small problems: every expert type,
random expert widths (f32/f16/bf16 1-300, block types 1-2 whole blocks), K
1-200, 1-40 experts, 1-8 used per token (distinct top-k routing, or every
slot on a few experts), 1-300 tokens, automatic plans.  Each case is
checked element by element against the oracle with the parity gate."""
import numpy as np
import pytest

from outer_product_gemm_amd import synth
from tests.test_gpu_id_back import _gpu, check_id, run_id  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu

TYPES = [synth.F32, synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0, synth.Q5_1,
         synth.Q8_0, synth.Q2_K, synth.Q3_K, synth.Q4_K, synth.Q5_K, synth.Q6_K]
PER_TYPE = 4


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    for a_type in TYPES:
        qk = synth.BLOCK_VALUES[a_type]
        for i in range(PER_TYPE):
            ne00 = int(rng.integers(1, 301)) if qk == 1 else qk * int(rng.integers(1, 3))
            K = int(rng.integers(1, 201))
            E = int(rng.integers(1, 41))
            n_used = int(rng.integers(1, min(8, E) + 1))
            n_tok = int(rng.integers(1, 301))
            skew = bool(i % 2) and E > 1   # every slot on at most 3 experts
            seed = int(rng.integers(0, 2 ** 31 - 1))
            out.append((a_type, ne00, K, E, n_used, n_tok, skew, seed))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%dx%d-E%d-u%d-t%d%s" % (
    synth.TYPE_NAMES[c[0]], c[1], c[2], c[3], c[4], c[5], "-skew" if c[6] else ""))
def test_id_back_random_small(case):
    a_type, ne00, K, E, n_used, n_tok, skew, seed = case
    inst = synth.make_moe_instance("rid", a_type, ne00, K, E, n_used, n_tok, seed)
    if skew:
        # the i-th used expert of every token is expert i mod 3 (distinct per
        # token when n_used <= 3, repeated otherwise: repeats are legal ids)
        inst.ids = (np.arange(n_used, dtype=np.int32)[None, :] % min(3, E)).repeat(n_tok, 0)
        inst.ids = np.ascontiguousarray(inst.ids)
    gpu, _ = run_id(inst)
    check_id(inst, gpu)
