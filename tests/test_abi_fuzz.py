"""Host-side validation under arbitrary arguments (no GPU: the plan entry
points never touch the device).  For random and adversarial ne/nb (negative,
zero, huge, overflowing products), type ids, kernel codes and pointers, the
library must return a documented status -- never crash -- and an accepted
problem must be self-consistent: its workgroup count fits the launch range,
and the tile and split report covers the problem."""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth

TYPE_IDS = [0, 1, 2, 3, 6, 7, 8, 10, 11, 12, 13, 14, 30]
KNOWN = set(B.STATUS) | {0}

extent = st.one_of(st.integers(-3, 3), st.integers(0, 600), st.integers(1, 1 << 20),
                   st.sampled_from([1 << 31, (1 << 31) - 1, 1 << 40, (1 << 62) + 1, -(1 << 62)]))
stride = st.one_of(st.integers(-64, 64), st.integers(0, 1 << 24),
                   st.sampled_from([0, 2, 4, 18, 34, 144, 1 << 33, (1 << 62) + 4, -(1 << 40)]))
ptr = st.sampled_from([0, 1, 2, 0x10000000, 0x10000002, 0x40000000000, 0x80000000000, (1 << 63) - 16])
type_id = st.one_of(st.sampled_from(TYPE_IDS), st.integers(-5, 40))
kernel = st.one_of(st.sampled_from([0, 1, 2, 3, 4]), st.integers(-3, 1 << 26))

SETTINGS = dict(max_examples=1500, deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow])


@pytest.fixture(scope="module", autouse=True)
def _lib():
    B.load_library()


@settings(**SETTINGS)
@given(st.lists(extent, min_size=12, max_size=12), st.lists(stride, min_size=12, max_size=12),
       type_id, ptr, ptr, ptr, kernel)
def test_out_prod_plan_never_crashes(ne, nb, a_type, a, b, d, k):
    st_ = B.plan_status(a, a_type, b, d, ne, nb, k)
    assert st_ in KNOWN
    if st_ == 0:
        p = B.out_prod_plan(a, a_type, b, d, ne, nb, k)
        assert 0 <= p["grid"] <= (1 << 31) - 1
        assert p["splits"] >= 1 and p["ksplit"] >= 0


@settings(**SETTINGS)
@given(st.sampled_from(TYPE_IDS), st.integers(1, 3), st.integers(0, 300), st.integers(1, 3000),
       st.integers(0, 300), st.integers(1, 4), st.integers(1, 4), st.booleans(),
       st.sampled_from([0, 1, 2]))
def test_valid_shapes_always_plan(a_type, blocks, w, n, K, ne02, d2, kt, fam):
    """Well-formed contiguous problems are always accepted by the automatic
    choice and by both forced families where they apply (K == 0 runs the
    zero kernel whatever the family), and the plan's workgroups cover the
    output."""
    qk = synth.BLOCK_VALUES[a_type]
    ne00 = blocks * qk if qk > 1 else max(1, w)
    ne, nb = synth.make_ne_nb(a_type, (ne00, K, ne02, 1), (n, K, ne02 * d2, 1), b_kt=kt)
    a, b, d = 0x10000000, 0x40000000000, 0x80000000000
    code = {0: B.KERNEL_AUTO, 1: B.KERNEL_TILED, 2: B.KERNEL_SKINNY}[fam]
    st_ = B.plan_status(a, a_type, b, d, ne, nb, code)
    if K == 0:
        assert st_ == 0 and B.out_prod_plan(a, a_type, b, d, ne, nb, code)["kernel_name"] == "zero"
        return
    if fam == 2 and a_type != synth.F32:
        assert B.STATUS.get(st_) == "E_KERNEL"
        return
    assert st_ == 0, (B.STATUS.get(st_), ne, nb)
    p = B.out_prod_plan(a, a_type, b, d, ne, nb, code)
    if p["kernel_name"] == "tiled":
        tiles = -(-ne00 // p["tile_m"]) * -(-n // p["tile_n"]) * ne02 * d2
        if p["swapped"]:
            tiles = -(-n // p["tile_m"]) * -(-ne00 // p["tile_n"]) * ne02 * d2
        assert p["grid"] == tiles * p["splits"]
    assert p["splits"] >= 1 and (p["splits"] - 1) * p["ksplit"] < K <= p["splits"] * p["ksplit"]


@settings(**SETTINGS)
@given(st.lists(extent, min_size=16, max_size=16), st.lists(stride, min_size=16, max_size=16),
       type_id, ptr, ptr, ptr, ptr, kernel)
def test_id_back_plan_never_crashes(ne, nb, a_type, a, g, ids, d, k):
    st_ = B.id_back_plan_status(a, a_type, g, ids, d, ne, nb, k)
    assert st_ in KNOWN
