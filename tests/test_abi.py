"""The C ABI on the host: the library loads, exports every declared symbol,
and refuses every contract violation with its status code before any HIP call
(so these run without a GPU).  Data pointers here are fake addresses that are
never dereferenced: out_prod_plan only checks them, and out_prod returns on
the failed check before touching the device."""
import os
import re

import pytest

from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A, BB, D = 0x10000000, 0x20000000, 0x30000000   # fake, 256-aligned, disjoint


def declared_functions():
    src = open(os.path.join(ROOT, "include", "outprod.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    lib = B.load_library()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    assert B.out_prod_version() == 3
    for code in [0] + list(B.STATUS):
        msg = B.out_prod_strerror(code)
        assert msg and msg != "unknown status"
    assert B.out_prod_strerror(-999) == "unknown status"


def base(a_type=synth.F32, a_ne=(8, 512, 1, 1), b_ne=(2560, 512, 1, 1)):
    ne, nb = synth.make_ne_nb(a_type, a_ne, b_ne)
    return list(ne), list(nb)


def plan(a_type, ne, nb, a=A, b=BB, d=D, kernel=0):
    return B.plan_status(a, a_type, b, d, ne, nb, kernel)


def test_valid_problem_plans():
    ne, nb = base()
    assert plan(synth.F32, ne, nb) == 0
    p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb)
    assert p["kernel_name"] == "skinny" and p["slices"] == 1 and p["flops"] == 2 * 8 * 2560 * 512


@pytest.mark.parametrize("mutate,code", [
    (lambda ne, nb: ne.__setitem__(5, 511), "E_K"),
    (lambda ne, nb: ne.__setitem__(8, 9), "E_DST_SHAPE"),
    (lambda ne, nb: ne.__setitem__(9, 2561), "E_DST_SHAPE"),
    (lambda ne, nb: ne.__setitem__(0, -1), "E_SHAPE"),
    (lambda ne, nb: nb.__setitem__(0, 8), "E_LAYOUT"),      # a not unit stride
    (lambda ne, nb: nb.__setitem__(4, 2048), "E_LAYOUT"),   # neither b dim contiguous
    (lambda ne, nb: nb.__setitem__(8, 8), "E_LAYOUT"),
    (lambda ne, nb: nb.__setitem__(5, 10242), "E_LAYOUT"),  # misaligned stride
    (lambda ne, nb: nb.__setitem__(9, 16), "E_LAYOUT"),     # dst rows overlap
    (lambda ne, nb: nb.__setitem__(1, -32), "E_LAYOUT"),
])
def test_contract_violations(mutate, code):
    ne, nb = base()
    mutate(ne, nb)
    assert B.STATUS[plan(synth.F32, ne, nb)] == code
    # out_prod itself returns the same status without touching the device
    assert B.STATUS[B.out_prod_status(A, synth.F32, BB, D, ne, nb)] == code


def test_broadcast_divisibility():
    ne, nb = base(a_ne=(128, 512, 4, 1), b_ne=(128, 512, 16, 1))
    assert plan(synth.F32, ne, nb) == 0
    assert B.out_prod_plan(A, synth.F32, BB, D, ne, nb)["dps2"] == 4
    ne, nb = base(a_ne=(128, 512, 3, 1), b_ne=(128, 512, 16, 1))
    assert B.STATUS[plan(synth.F32, ne, nb)] == "E_BCAST"
    ne, nb = base(a_ne=(128, 512, 1, 2), b_ne=(128, 512, 1, 3))
    assert B.STATUS[plan(synth.F32, ne, nb)] == "E_BCAST"


def test_type_and_block_width():
    ne, nb = base()
    for bad in (4, 5, 9, 15, 16, 29, 31, 99, -1):
        assert B.STATUS[plan(bad, ne, nb)] == "E_TYPE", bad
    ne, nb = base(synth.Q8_0, a_ne=(64, 512, 1, 1))
    assert plan(synth.Q8_0, ne, nb) == 0
    ne[0] = ne[8] = 48
    assert B.STATUS[plan(synth.Q8_0, ne, nb)] == "E_QK"
    ne, nb = base(synth.Q4_K, a_ne=(512, 64, 1, 1), b_ne=(16, 64, 1, 1))
    assert plan(synth.Q4_K, ne, nb) == 0
    ne[0] = ne[8] = 384
    assert B.STATUS[plan(synth.Q4_K, ne, nb)] == "E_QK"
    # quant blocks must be addressed with their byte size as nb[0]
    ne, nb = base(synth.Q4_K, a_ne=(512, 64, 1, 1), b_ne=(16, 64, 1, 1))
    nb[0] = 4
    assert B.STATUS[plan(synth.Q4_K, ne, nb)] == "E_LAYOUT"


def test_pointer_checks():
    ne, nb = base()
    assert B.STATUS[plan(synth.F32, ne, nb, a=0)] == "E_NULL"
    assert B.STATUS[plan(synth.F32, ne, nb, b=0)] == "E_NULL"
    assert B.STATUS[plan(synth.F32, ne, nb, d=0)] == "E_NULL"
    assert B.STATUS[plan(synth.F32, ne, nb, b=BB + 2)] == "E_LAYOUT"
    assert B.STATUS[plan(synth.F32, ne, nb, d=BB + 4096)] == "E_ALIAS"   # dst inside b
    assert B.STATUS[plan(synth.F32, ne, nb, d=A + 4)] == "E_ALIAS"
    # q8_0 rows are 2-byte aligned: an odd address is refused, an even one is fine
    ne, nb = base(synth.Q8_0, a_ne=(64, 512, 1, 1))
    assert B.STATUS[plan(synth.Q8_0, ne, nb, a=A + 1)] == "E_LAYOUT"
    assert plan(synth.Q8_0, ne, nb, a=A + 2) == 0


def test_empty_and_zero_k():
    ne, nb = base(b_ne=(0, 512, 1, 1))
    assert B.out_prod_plan(A, synth.F32, BB, D, ne, nb)["kernel_name"] == "none"
    # empty dst needs no pointers at all
    assert plan(synth.F32, ne, nb, a=0, b=0, d=0) == 0
    ne, nb = base(a_ne=(8, 0, 1, 1), b_ne=(2560, 0, 1, 1))
    p = B.out_prod_plan(0, synth.F32, 0, D, ne, nb)
    assert p["kernel_name"] == "zero"


def test_range_limit():
    ne, nb = base(b_ne=(1 << 31, 1, 1, 1), a_ne=(8, 1, 1, 1))
    assert B.STATUS[plan(synth.F32, ne, nb)] == "E_RANGE"


def test_kernel_choice_on_workloads():
    want = {
        "lora_r8_single": "skinny", "lora_r4_2560": "skinny", "lora_r24_9216": "skinny",
        "deltanet_bcast": "skinny", "q8_0_5120": "tiled", "q4_K_5120x17408": "tiled",
        "q4_K_17408x5120": "tiled",
    }
    for name, kern in want.items():
        a_type, a_ne, b_ne = synth.WORKLOADS[name][:3]
        ne, nb = synth.make_ne_nb(a_type, a_ne, b_ne)
        p = B.out_prod_plan(A, a_type, 0x40000000000, 0x80000000000, ne, nb)
        assert p["kernel_name"] == kern, name
        assert p["grid"] >= 1


def test_tile_choice_at_the_27B_shapes():
    """The planner's measured tile choices at m5120 k17408 n1024 (one launch
    per CU round): the 80 x 256 tile (configuration 14, half the a decode per
    flop) for the K-quants with sub-block scales, 160 x 128 (configuration
    8) for the types whose decode is cheap; 272 x 128 with loader waves for
    m17408 k5120 (configuration 19, or 20 -- loads two stages ahead -- for
    q4_0, q5_0 and q8_0); the K-contiguous 27B input
    gradient like its type."""
    for name, cfg in (("q4_K_5120x17408", 14), ("q6_K_5120x17408", 14), ("q3_K_5120x17408", 14),
                      ("q5_K_5120x17408", 14), ("f32_5120x17408", 8), ("f16_5120x17408", 8),
                      ("q8_0_5120x17408", 8), ("q4_0_5120x17408", 8), ("q4_K_17408x5120", 19),
                      ("q8_0_5120", 8), ("lora27B_dxW", 14)):
        inst_spec = synth.WORKLOADS[name]
        a_type, a_ne, b_ne = inst_spec[:3]
        kt = inst_spec[7] if len(inst_spec) > 7 else False
        ne, nb = synth.make_ne_nb(a_type, a_ne, b_ne, kt)
        p = B.out_prod_plan(A, a_type, 0x40000000000, 0x80000000000, ne, nb)
        assert p["kernel_name"] == "tiled" and p["variant"] == cfg and p["splits"] == 1, (name, p)
        assert p["grid"] == (256 if cfg != 19 else 512), (name, p)
    # m17408 k5120 n1024 for each type: 19, or 20 for q4_0, q5_0, q8_0
    for t in synth.TYPE_NAMES:
        ne, nb = synth.make_ne_nb(t, (17408, 5120, 1, 1), (1024, 5120, 1, 1))
        p = B.out_prod_plan(A, t, 0x40000000000, 0x80000000000, ne, nb)
        want = 20 if t in (synth.Q4_0, synth.Q5_0, synth.Q8_0) else 19
        assert p["variant"] == want and p["block"] == 1024 and p["lds_bytes"] == 159744, (t, p)


def test_forced_kernels():
    ne, nb = base()
    assert B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.KERNEL_TILED)["kernel_name"] == "tiled"
    ne, nb = base(synth.Q8_0, a_ne=(64, 512, 1, 1))
    assert B.STATUS[plan(synth.Q8_0, ne, nb, kernel=B.KERNEL_SKINNY)] == "E_KERNEL"
    ne, nb = base(a_ne=(33, 512, 1, 1))
    p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.KERNEL_SKINNY)
    assert p["kernel_name"] == "skinny" and p["tile_m"] == 32 and p["tile_n"] == 32 and p["grid"] == 2 * 80
    assert B.STATUS[plan(synth.F32, ne, nb, kernel=7)] == "E_KERNEL"
    for cfg in range(13):
        p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.kernel_code(B.KERNEL_SKINNY, cfg))
        assert p["kernel_name"] == "skinny" and p["variant"] == cfg
    assert B.STATUS[plan(synth.F32, ne, nb, kernel=B.kernel_code(B.KERNEL_SKINNY, 13))] == "E_KERNEL"
    # every tiled configuration can be forced; an unknown one is refused
    for cfg in B.TILED_CONFIGS:
        p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.kernel_code(B.KERNEL_TILED, cfg))
        assert p["kernel_name"] == "tiled" and p["variant"] == cfg
    # 15 to 18 are built for the grouped MUL_MAT_ID_BACK kernel only
    for cfg in (15, 16, 17, 18, 21, 40):
        assert B.STATUS[plan(synth.F32, ne, nb, kernel=B.kernel_code(B.KERNEL_TILED, cfg))] == "E_KERNEL"


def test_k_contiguous_b_layout():
    """b as a transposed view (K contiguous) is accepted by both families;
    wide-strip column configurations refuse it."""
    ne, nb = synth.make_ne_nb(synth.Q4_K, (512, 64, 1, 1), (16, 64, 1, 1), b_kt=True)
    assert nb[4] == 4 * 64 and nb[5] == 4
    p = B.out_prod_plan(A, synth.Q4_K, BB, D, ne, nb)
    assert p["kernel_name"] == "tiled"
    ne, nb = synth.make_ne_nb(synth.F32, (8, 512, 1, 1), (2560, 512, 1, 1), b_kt=True)
    p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb)
    assert p["kernel_name"] == "skinny" and p["tile_n"] == 16
    assert B.STATUS[plan(synth.F32, ne, nb, kernel=B.kernel_code(B.KERNEL_SKINNY, 2))] == "E_KERNEL"
    assert plan(synth.F32, ne, nb, kernel=B.kernel_code(B.KERNEL_SKINNY, 6)) == 0
    # b's extent with the K-contiguous layout: dst right after b's last byte is fine,
    # dst on b's last float aliases
    last = BB + 4 * 512 * 2560
    assert plan(synth.F32, ne, nb, d=last) == 0
    assert B.STATUS[plan(synth.F32, ne, nb, d=last - 4)] == "E_ALIAS"


def test_narrow_b_runs_operand_swapped():
    """A narrow f32 b with a wide f32 a (a LoRA down-projection's gradient
    out_prod(x, grad_h)) runs the column kernel on the swapped problem."""
    ne, nb = synth.make_ne_nb(synth.F32, (2560, 512, 1, 1), (8, 512, 1, 1))
    p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb)
    assert p["kernel_name"] == "skinny" and p["swapped"] == 1
    ne, nb = synth.make_ne_nb(synth.F32, (2560, 512, 1, 1), (8, 512, 1, 1), b_kt=True)
    assert B.out_prod_plan(A, synth.F32, BB, D, ne, nb)["swapped"] == 0
    ne, nb = synth.make_ne_nb(synth.Q8_0, (2560, 512, 1, 1), (8, 512, 1, 1))
    assert B.out_prod_plan(A, synth.Q8_0, BB, D, ne, nb)["swapped"] == 0


def test_split_k_plans():
    """Long-K problems with few output tiles split K; the plan reports the
    ranges and the workspace; forced split counts are honoured or refused."""
    # 4B-scale input gradient through a frozen q4_K weight: 64 tiles of 160 x 128
    ne, nb = synth.make_ne_nb(synth.Q4_K, (2560, 9216, 1, 1), (512, 9216, 1, 1), b_kt=True)
    p = B.out_prod_plan(A, synth.Q4_K, 0x40000000000, 0x80000000000, ne, nb)
    assert p["kernel_name"] == "tiled" and p["splits"] > 1
    assert p["ksplit"] % 64 == 0 and (p["splits"] - 1) * p["ksplit"] < 9216 <= p["splits"] * p["ksplit"]
    assert p["workspace_bytes"] == p["splits"] * 2560 * 512 * 4 <= 64 << 20
    tiles = -(-2560 // p["tile_m"]) * -(-512 // p["tile_n"])
    assert p["grid"] == tiles * p["splits"]
    # rank-8 gradient with a long K and few column strips
    ne, nb = synth.make_ne_nb(synth.F32, (8, 9216, 1, 1), (512, 9216, 1, 1), b_kt=True)
    p = B.out_prod_plan(A, synth.F32, 0x40000000000, 0x80000000000, ne, nb)
    assert p["kernel_name"] == "skinny" and p["splits"] > 1 and p["ksplit"] >= 256
    # the 27B q4_K products fill the chip unsplit
    for name in ("q4_K_5120x17408", "q4_K_17408x5120", "q8_0_5120", "lora_r8_9216"):
        a_type, a_ne, b_ne = synth.WORKLOADS[name][:3]
        ne, nb = synth.make_ne_nb(a_type, a_ne, b_ne)
        p = B.out_prod_plan(A, a_type, 0x40000000000, 0x80000000000, ne, nb)
        assert p["splits"] == 1 and p["workspace_bytes"] == 0 and p["ksplit"] == a_ne[1], name
    # forced split counts (any row count), refused when impossible
    ne, nb = base(a_ne=(40, 100, 1, 1), b_ne=(70, 100, 1, 1))
    for fam in (B.KERNEL_TILED, B.KERNEL_SKINNY):
        p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.kernel_code(fam, None, 3))
        assert p["splits"] == 3 and p["ksplit"] == 34 and p["workspace_bytes"] == 3 * 40 * 70 * 4
        p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.kernel_code(fam, None, 1))
        assert p["splits"] == 1 and p["workspace_bytes"] == 0
        assert B.STATUS[plan(synth.F32, ne, nb, kernel=B.kernel_code(fam, None, 101))] == "E_KERNEL"
    # 100 rows in 40 ranges: ceil(100/40) = 3 rows each, so 34 ranges
    p = B.out_prod_plan(A, synth.F32, BB, D, ne, nb, B.kernel_code(B.KERNEL_TILED, None, 40))
    assert p["ksplit"] == 3 and p["splits"] == 34
    # partials beyond the 64 MiB workspace
    ne, nb = base(a_ne=(4096, 100, 1, 1), b_ne=(4096, 100, 1, 1))
    assert B.STATUS[plan(synth.F32, ne, nb, kernel=B.kernel_code(B.KERNEL_TILED, None, 2))] == "E_KERNEL"
    # split bits need a forced family; bits above 23 are refused
    assert B.STATUS[plan(synth.F32, ne, nb, kernel=B.kernel_code(B.KERNEL_AUTO, None, 2))] == "E_KERNEL"
    assert B.STATUS[plan(synth.F32, ne, nb, kernel=1 << 24)] == "E_KERNEL"


ALL_TYPES = [synth.F32, synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0, synth.Q5_1,
             synth.Q8_0, synth.Q2_K, synth.Q3_K, synth.Q4_K, synth.Q5_K, synth.Q6_K]


@pytest.mark.parametrize("a_type", ALL_TYPES)
def test_every_a_type_plans(a_type):
    """Every type of the frozen-weight set is accepted with its block size as
    nb[0] and whole blocks; widths off the block grid, a wrong nb[0], and
    strides or pointers below the type's alignment are refused."""
    qk, bb = synth.BLOCK_VALUES[a_type], synth.BLOCK_BYTES[a_type]
    width = 512
    ne, nb = base(a_type, a_ne=(width, 64, 1, 1), b_ne=(96, 64, 1, 1))
    assert nb[0] == bb and nb[1] == width // qk * bb
    p = B.out_prod_plan(A, a_type, BB, D, ne, nb)
    expect = "skinny" if a_type == synth.F32 else "tiled"
    assert p["kernel_name"] == expect and p["flops"] == 2 * width * 96 * 64
    if qk > 1:
        ne2 = list(ne)
        ne2[0] = ne2[8] = width - qk // 2
        assert B.STATUS[plan(a_type, ne2, nb)] == "E_QK"
    nb2 = list(nb)
    nb2[0] = bb + 2
    assert B.STATUS[plan(a_type, ne, nb2)] == "E_LAYOUT"
    al = 4 if bb % 4 == 0 else 2
    nb2 = list(nb)
    nb2[1] += al        # row stride of the type's alignment: accepted
    assert plan(a_type, ne, nb2) == 0
    nb2[1] += 1         # odd stride: refused
    assert B.STATUS[plan(a_type, ne, nb2)] == "E_LAYOUT"
    assert plan(a_type, ne, nb, a=A + al) == 0
    if al == 4:
        assert B.STATUS[plan(a_type, ne, nb, a=A + 2)] == "E_LAYOUT"
    assert B.STATUS[plan(a_type, ne, nb, a=A + 1)] == "E_LAYOUT"
    # the skinny kernel is f32 only
    if a_type != synth.F32:
        assert B.STATUS[plan(a_type, ne, nb, kernel=B.KERNEL_SKINNY)] == "E_KERNEL"


# ---------------------------------------------------------------- MUL_MAT_ID_BACK

G_ = 0x50000000000
I_ = 0x60000000000


def id_plan(inst, a=A, g=G_, ids=I_, d=D, ne=None, nb=None, kernel=0):
    return B.id_back_plan_status(a, inst.a_type, g, ids, d, ne or inst.ne, nb or inst.nb, kernel)


def test_id_back_automatic_tiles():
    """The grouped kernel's automatic tiles on the 64-expert shapes: 128 x 96
    slot tiles, with 32-row stages where fewer than three 8-wave workgroups
    per CU would be resident (the down-projection gradient's 512 tiles)."""
    for name, cfg, bk in (("moe_up_back_q4_K", 17, 16), ("moe_down_back_q4_K", 18, 32)):
        inst = synth.moe_workload(name)
        p = B.out_prod_id_back_plan(A, inst.a_type, G_, I_, D, inst.ne, inst.nb)
        assert (p["variant"], p["tile_m"], p["tile_n"], p["tile_k"], p["block"]) == (cfg, 128, 96, bk, 512), (name, p)
    # few tokens: slot tiles stay small (64 x 64)
    inst = synth.make_moe_instance("few", synth.Q4_K, 2560, 1024, 64, 8, 16, 1)
    p = B.out_prod_id_back_plan(A, inst.a_type, G_, I_, D, inst.ne, inst.nb)
    assert p["tile_n"] <= 80, p


def test_id_back_plans_and_refusals():
    inst = synth.make_moe_instance("abi", synth.Q4_K, 512, 96, 8, 2, 40, 1)
    p = B.out_prod_id_back_plan(A, synth.Q4_K, G_, I_, D, inst.ne, inst.nb)
    assert p["kernel_name"] == "tiled" and p["slices"] == 80 and p["flops"] == 2 * 512 * 96 * 80
    assert p["workspace_bytes"] > 0 and p["grid"] >= 1
    for cfg in (0, 1, 2, 4, 8, 10, 11, 12, 13, 15, 16, 17, 18):
        q = B.out_prod_id_back_plan(A, synth.Q4_K, G_, I_, D, inst.ne, inst.nb,
                                    B.kernel_code(B.KERNEL_TILED, cfg))
        assert q["variant"] == cfg
    for cfg in (3, 19, 20):  # OUT_PROD-only configurations
        assert B.STATUS[id_plan(inst, kernel=B.kernel_code(B.KERNEL_TILED, cfg))] == "E_KERNEL"
    assert B.STATUS[id_plan(inst, kernel=B.KERNEL_SKINNY)] == "E_KERNEL"
    assert B.STATUS[id_plan(inst, kernel=B.kernel_code(B.KERNEL_TILED, None, 2))] == "E_KERNEL"
    ne = list(inst.ne)
    ne[4] = 95
    assert B.STATUS[id_plan(inst, ne=ne)] == "E_K"
    ne = list(inst.ne)
    ne[13] = 3
    assert B.STATUS[id_plan(inst, ne=ne)] == "E_DST_SHAPE"
    ne = list(inst.ne)
    ne[8] = 3
    assert B.STATUS[id_plan(inst, ne=ne)] == "E_SHAPE"
    ne = list(inst.ne)
    ne[0] = ne[12] = 384
    assert B.STATUS[id_plan(inst, ne=ne)] == "E_QK"
    nb = list(inst.nb)
    nb[4] = 8           # g must be K-contiguous
    assert B.STATUS[id_plan(inst, nb=nb)] == "E_LAYOUT"
    nb = list(inst.nb)
    nb[13] = 4 * 500    # dst rows overlap
    assert B.STATUS[id_plan(inst, nb=nb)] == "E_LAYOUT"
    assert B.STATUS[id_plan(inst, ids=0)] == "E_NULL"
    assert B.STATUS[id_plan(inst, ids=I_ + 2)] == "E_LAYOUT"
    assert B.STATUS[id_plan(inst, d=G_ + 64)] == "E_ALIAS"
    assert B.STATUS[id_plan(inst, d=I_)] == "E_ALIAS"
    big = synth.moe_ne_nb(synth.Q4_K, 256, 8, 513, 2, 4)
    assert B.STATUS[B.id_back_plan_status(A, synth.Q4_K, G_, I_, D, *big)] == "E_RANGE"
    # nothing to do: no tokens; K == 0: zeros
    ne0, nb0 = synth.moe_ne_nb(synth.F32, 16, 8, 4, 2, 0)
    assert B.out_prod_id_back_plan(A, synth.F32, G_, I_, D, ne0, nb0)["kernel_name"] == "none"
    ne0, nb0 = synth.moe_ne_nb(synth.F32, 16, 0, 4, 2, 3)
    assert B.out_prod_id_back_plan(A, synth.F32, G_, I_, D, ne0, nb0)["kernel_name"] == "zero"
    assert B.out_prod_id_back_plan(0, synth.F32, 0, 0, D, ne0, nb0)["kernel_name"] == "zero"


@pytest.mark.parametrize("a_type", ALL_TYPES)
def test_id_back_every_type_plans(a_type):
    qk = synth.BLOCK_VALUES[a_type]
    inst_ne, inst_nb = synth.moe_ne_nb(a_type, 256 if qk > 1 else 100, 64, 4, 2, 8)
    p = B.out_prod_id_back_plan(A, a_type, G_, I_, D, inst_ne, inst_nb)
    assert p["kernel_name"] == "tiled"


def test_tile_order_reported_and_forced():
    """The tiled kernel's tile order within a slice (groups of group_m tiles
    along i0, i0 fastest inside a group) is reported by the plan and chosen
    per shape: i0 fastest for m5120 k17408 (one round of tiles per XCD, every
    XCD's tiles share one b strip), groups of 8 for m17408 k5120 (two rounds:
    8 a strips and 4 b strips per round).  It can be forced (a value past the
    tiles along i0 means i0 fastest); other families refuse it and report 0."""
    for name, want in (("q4_K_5120x17408", 64), ("q4_K_17408x5120", 8)):
        a_type, a_ne, b_ne = synth.WORKLOADS[name][:3]
        ne, nb = synth.make_ne_nb(a_type, a_ne, b_ne)
        p = B.out_prod_plan(A, a_type, 0x40000000000, 0x80000000000, ne, nb)
        assert p["kernel_name"] == "tiled" and p["group_m"] == want, (name, p)
        tiles_m = -(-a_ne[0] // p["tile_m"])
        for g, expect in ((1, 1), (3, 3), (127, min(127, tiles_m))):
            code = B.kernel_code(B.KERNEL_TILED, p["variant"], None, g)
            q = B.out_prod_plan(A, a_type, 0x40000000000, 0x80000000000, ne, nb, code)
            assert q["group_m"] == expect and q["variant"] == p["variant"] and q["grid"] == p["grid"]
    ne, nb = base()
    assert B.out_prod_plan(A, synth.F32, BB, D, ne, nb)["group_m"] == 0
    for fam in (B.KERNEL_SKINNY, B.KERNEL_AUTO):
        code = B.kernel_code(fam, None, None, 2)
        assert B.STATUS[plan(synth.F32, ne, nb, kernel=code)] == "E_KERNEL"


def test_tensor_helpers_refuse_wrong_dtypes_and_devices():
    """out_prod_tensors / tensor_ne_nb describe memory from each tensor's
    dtype; a b or out that is not float32, an a whose dtype does not match
    a_type, and tensors off the GPU are refused with ValueError before
    anything reaches the library."""
    import torch
    a = torch.zeros(512, 8)
    b = torch.zeros(512, 2560)
    out = torch.zeros(2560, 8)
    ne, nb = B.tensor_ne_nb(a, synth.F32, b, out)
    assert ne == [8, 512, 1, 1, 2560, 512, 1, 1, 8, 2560, 1, 1]
    assert nb[:2] == [4, 32] and nb[4:6] == [4, 4 * 2560] and nb[8:10] == [4, 32]
    for bad_b in (b.half(), b.bfloat16(), b.double()):
        with pytest.raises(ValueError, match="b must be float32"):
            B.tensor_ne_nb(a, synth.F32, bad_b, out)
    with pytest.raises(ValueError, match="out must be float32"):
        B.tensor_ne_nb(a, synth.F32, b, out.half())
    with pytest.raises(ValueError, match="a has dtype"):
        B.tensor_ne_nb(a.half(), synth.F32, b, out)
    with pytest.raises(ValueError, match="a has dtype"):
        B.tensor_ne_nb(a, synth.F16, b, out)
    with pytest.raises(ValueError, match="a has dtype"):
        B.tensor_ne_nb(a, synth.Q4_K, b, out)
    # f16 a: byte strides from the 2-byte element size
    ne, nb = B.tensor_ne_nb(a.half(), synth.F16, b, out)
    assert nb[:2] == [2, 16]
    # quantized a as packed bytes
    qa = torch.zeros(512, 144, dtype=torch.uint8)
    ne, nb = B.tensor_ne_nb(qa, synth.Q4_K, b, torch.zeros(2560, 256))
    assert ne[0] == 256 and nb[:2] == [144, 144]
    with pytest.raises(ValueError, match="GPU tensor"):
        B.out_prod_tensors(a, synth.F32, b, out)
