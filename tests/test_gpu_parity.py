"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Gate (per element): no NaN/Inf, |gpu - ref| <= 1e-5 * sum_k |a||b|.  Integer
inputs, one-hot b and K = 1 are checked bit for bit.  Sizes: small ragged
shapes spanning several tiles for both kernels; every workload at full size
in the launch configuration the benchmark uses, with the oracle on sampled
output columns where the full oracle would take too long.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield


def seed_of(*parts):
    return zlib.crc32(repr(parts).encode()) & 0x7FFFFFFF


def check_case(inst, kernel=0, cols=None):
    G.log("case", inst.name, synth.TYPE_NAMES[inst.a_type], inst.ne[:8], "kernel", kernel)
    gpu = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb, kernel)
    if cols is None:
        ref, den = oracle.out_prod(inst.a, inst.a_type, inst.b, inst.ne, inst.nb)
        res = oracle.check(gpu, ref, den, TOL)
        assert np.isfinite(gpu).all()
    else:
        ref, den = oracle.out_prod(inst.a, inst.a_type, inst.b, inst.ne, inst.nb, cols=cols)
        g = np.stack([gpu[i3, i2, i1] for i1, i2, i3 in cols])
        res = oracle.check(g, ref, den, TOL)
        assert np.isfinite(gpu).all(), "NaN/Inf in the full GPU output"
    G.log("   ", res)
    assert res["ok"], res
    return gpu


SMALL = [
    # (a_type, a_ne, b_ne, kernel)
    (synth.F32, (1, 7, 1, 1), (5, 7, 1, 1), 0),
    (synth.F32, (4, 100, 1, 1), (33, 100, 1, 1), 0),
    (synth.F32, (8, 512, 1, 1), (100, 512, 1, 1), 0),
    (synth.F32, (13, 33, 2, 1), (37, 33, 4, 1), 0),
    (synth.F32, (24, 65, 1, 2), (300, 65, 1, 4), 0),
    (synth.F32, (32, 511, 1, 1), (17, 511, 1, 1), 0),
    (synth.F32, (16, 3, 1, 1), (16, 3, 1, 1), 0),
    (synth.F32, (33, 17, 1, 1), (1, 17, 1, 1), 0),
    (synth.F32, (130, 100, 2, 1), (129, 100, 4, 1), 0),
    (synth.F32, (257, 40, 1, 2), (300, 40, 1, 2), 0),
    (synth.F32, (128, 512, 1, 1), (128, 512, 1, 1), 0),
    (synth.F32, (200, 1, 1, 1), (150, 1, 1, 1), 0),
    (synth.F32, (8, 512, 1, 1), (100, 512, 1, 1), B.KERNEL_TILED),
    (synth.F32, (24, 65, 1, 2), (300, 65, 1, 4), B.KERNEL_TILED),
    (synth.F32, (5, 31, 3, 1), (70, 31, 6, 1), B.KERNEL_TILED),
    (synth.Q8_0, (32, 1, 1, 1), (7, 1, 1, 1), 0),
    (synth.Q8_0, (160, 33, 1, 1), (130, 33, 1, 1), 0),
    (synth.Q8_0, (288, 300, 2, 1), (70, 300, 4, 1), 0),
    (synth.Q4_K, (256, 1, 1, 1), (5, 1, 1, 1), 0),
    (synth.Q4_K, (512, 17, 1, 1), (130, 17, 1, 1), 0),
    (synth.Q4_K, (768, 70, 1, 2), (129, 70, 3, 2), 0),
]


@pytest.mark.parametrize("a_type,a_ne,b_ne,kernel", SMALL)
def test_small_ragged(a_type, a_ne, b_ne, kernel):
    inst = synth.make_instance("small", a_type, a_ne, b_ne, seed_of(a_type, a_ne, b_ne))
    check_case(inst, kernel)


@pytest.mark.parametrize("cfg", B.TILED_CONFIGS)
def test_every_tiled_configuration(cfg):
    """Each tiled configuration, forced, on ragged shapes of every a type
    (partial tiles in i0, i1 and K, broadcast slices)."""
    code = B.kernel_code(B.KERNEL_TILED, cfg)
    for a_type, a_ne, b_ne in ((synth.F32, (300, 45, 2, 1), (290, 45, 4, 1)),
                               (synth.Q8_0, (352, 70, 1, 1), (150, 70, 1, 1)),
                               (synth.Q4_K, (768, 37, 1, 2), (141, 37, 1, 2))):
        inst = synth.make_instance("cfg%d" % cfg, a_type, a_ne, b_ne, seed_of(cfg, a_type))
        check_case(inst, code)


@pytest.mark.parametrize("cfg", range(13))
def test_every_column_configuration(cfg):
    """Each column-kernel configuration, forced, on ragged f32 shapes (partial
    column strips, i0 blocks, K not a multiple of the wave steps, a column
    count that is not a multiple of 4, and b 4 bytes off a 16-byte boundary so
    that vector loads are off)."""
    code = B.kernel_code(B.KERNEL_SKINNY, cfg)
    for a_ne, b_ne in (((8, 517, 1, 1), (333, 517, 1, 1)), ((24, 130, 2, 1), (70, 130, 4, 1)),
                       ((50, 77, 1, 1), (45, 77, 1, 1)), ((3, 1100, 1, 1), (1030, 1100, 1, 1)),
                       ((24, 512, 1, 1), (640, 512, 1, 1)), ((30, 520, 1, 1), (96, 520, 1, 1))):
        inst = synth.make_instance("col%d" % cfg, synth.F32, a_ne, b_ne, seed_of(cfg, a_ne))
        check_case(inst, code)
    inst = synth.make_instance("colmis%d" % cfg, synth.F32, (8, 300, 1, 1), (200, 300, 1, 1), cfg)
    gpu = G.run(inst.a, synth.F32, inst.b, inst.ne, inst.nb, code, b_off=4)
    ref, den = oracle.out_prod(inst.a, synth.F32, inst.b, inst.ne, inst.nb)
    assert oracle.check(gpu, ref, den, TOL)["ok"]


def test_rank1_K1_bit_exact():
    """K = 1: dst = RN32(a[i0]*b[i1]) exactly, on both kernels."""
    for kernel, ne00 in ((B.KERNEL_SKINNY, 8), (B.KERNEL_TILED, 8), (B.KERNEL_TILED, 200)):
        inst = synth.make_instance("k1", synth.F32, (ne00, 1, 1, 1), (300, 1, 1, 1), 77)
        gpu = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb, kernel)
        expect = (inst.b[0, 0, 0][:, None].astype(np.float64) * inst.a[0, 0, 0][None, :]).astype(np.float32)
        assert np.array_equal(gpu[0, 0], expect)


# The benchmarked q8_0 and q4_K launches: their whole output is checked
# (the oracle needs a few seconds per launch on the host's cores).
WHOLE_OUTPUT = ("q8_0_5120", "q4_K_5120x17408", "q4_K_17408x5120", "q4_K_5120x5120")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_size(name):
    """Every workload at its full size, auto kernel choice (the bench's launch);
    every dst element of the q8_0 and q4_K 27B launches, sampled dst columns of
    the other 5120 x 17408 type-sweep launches."""
    inst = synth.workload(name)
    big = inst.ne[0] * inst.ne[1] * inst.ne[4] > 5e9 and name not in WHOLE_OUTPUT
    cols = None
    if big:
        rng = np.random.default_rng(seed_of(name))
        n = inst.ne[4]
        pick = sorted(set([0, n - 1, n // 2] + list(rng.choice(n, 13, replace=False))))
        cols = np.array([[i1, 0, 0] for i1 in pick])
    check_case(inst, 0, cols)


def _int_f32(rng, shape, lim=16):
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float32)


@pytest.mark.parametrize("a_ne,b_ne,kernel", [
    ((24, 512, 1, 1), (9216, 512, 1, 1), 0),         # skinny at the rank-24 shape
    ((128, 512, 4, 1), (128, 512, 16, 1), 0),        # broadcast shape
    ((256, 17408, 1, 1), (128, 17408, 1, 1), 0),     # long K: |sum| <= 4.46e6 < 2^24
])
def test_integer_exact_f32(a_ne, b_ne, kernel):
    rng = np.random.default_rng(seed_of("int", a_ne))
    ne, nb = synth.make_ne_nb(synth.F32, a_ne, b_ne)
    a = _int_f32(rng, (a_ne[3], a_ne[2], a_ne[1], a_ne[0]))
    b = _int_f32(rng, (b_ne[3], b_ne[2], b_ne[1], b_ne[0]))
    gpu = G.run(a, synth.F32, b, ne, nb, kernel)
    ref, _ = oracle.out_prod(a, synth.F32, b, ne, nb)
    assert np.array_equal(gpu, ref.astype(np.float32))


@pytest.mark.parametrize("name", ["q8_0_5120", "q4_K_5120x17408", "q4_K_17408x5120"])
def test_integer_exact_quant(name):
    """d = dmin = 1 and b in {-1, 0, 1}: every partial sum is an integer below
    2^24, so the GPU must equal the oracle bit for bit at the full shape, on
    every dst element."""
    a_type, a_ne, b_ne = synth.WORKLOADS[name][:3]
    rng = synth.rng_for(seed_of("intq", name))
    one = int(synth.fp16_bits([1.0])[0])
    nrows = a_ne[1]
    if a_type == synth.Q8_0:
        a = synth.q8_0_rows(rng, nrows, a_ne[0], d_bits=one)
    else:
        a = synth.q4_K_rows(rng, nrows, a_ne[0], d_bits=one, dmin_bits=one)
    b = rng.integers(-1, 2, size=(1, 1, b_ne[1], b_ne[0])).astype(np.float32)
    ne, nb = synth.make_ne_nb(a_type, a_ne, b_ne)
    G.log("int-exact", name)
    gpu = G.run(a, a_type, b, ne, nb)
    ref, _ = oracle.out_prod(a, a_type, b, ne, nb)
    assert np.array_equal(gpu, ref.astype(np.float32))


@pytest.mark.parametrize("name", ["q8_0_5120", "q4_K_5120x17408", "q4_K_17408x5120"])
def test_dequant_bit_exact_one_hot(name):
    """One-hot b picks row k of a into dst column i1, so dst = the kernel's own
    dequantized values.  Every row of a is covered, at the full shape, and
    must equal the oracle's decode bit for bit (as values: -0 == +0)."""
    inst = synth.workload(name)
    K, M, N = inst.ne[1], inst.ne[0], inst.ne[4]
    rowb = inst.a.shape[-1]
    expect = oracle.dequant_rows(inst.a.reshape(-1), inst.a_type, M, K, rowb)
    a_d = G.to_dev(inst.a.reshape(-1))
    out = torch.empty((N, M), dtype=torch.float32, device="cuda:0")
    ne, nb = inst.ne, inst.nb
    stream = torch.cuda.current_stream().cuda_stream
    for start in range(0, K, N):
        rows = np.arange(start, min(K, start + N))
        b_d = torch.zeros((K, N), dtype=torch.float32, device="cuda:0")
        cols = torch.arange(rows.size, device="cuda:0")
        b_d[torch.from_numpy(rows).to("cuda:0"), cols] = 1.0
        out.fill_(float("nan"))
        B.out_prod(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), out.data_ptr(), ne, nb, stream)
        got = out[: rows.size].cpu().numpy()
        assert np.array_equal(got, expect[rows]), (name, start)


def test_deterministic_repeat():
    for name in ("deltanet_bcast", "lora_r24_9216", "q8_0_5120"):
        inst = synth.workload(name)
        g1 = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb)
        g2 = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb)
        assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32)), name


def test_broadcast_invariant_gpu():
    """Slices sharing i2/dps2 with identical b slices are bit-identical, and
    each equals a one-slice call on (a[:,:,i2/dps2], b[:,:,i2]).  The split of
    K depends on the launch size (a lone slice leaves CUs idle and is split),
    so both calls pin the column kernel without a split."""
    inst = synth.workload("deltanet_bcast")
    b = inst.b.copy()
    b[0, 1] = b[0, 0]
    b[0, 6] = b[0, 0]   # another a slice (6 // 4 = 1)
    code = B.kernel_code(B.KERNEL_SKINNY, None, 1)
    gpu = G.run(inst.a, inst.a_type, b, inst.ne, inst.nb, code)
    assert np.array_equal(gpu[0, 0], gpu[0, 1])
    assert not np.array_equal(gpu[0, 0], gpu[0, 6])
    ne1, nb1 = synth.make_ne_nb(synth.F32, (128, 512, 1, 1), (128, 512, 1, 1))
    for i2 in (0, 5, 15):
        one = G.run(np.ascontiguousarray(inst.a[:, i2 // 4]), synth.F32,
                    np.ascontiguousarray(b[:, i2]), ne1, nb1, code)
        assert np.array_equal(one[0, 0], gpu[0, i2])


def test_strided_views_and_misalignment():
    """Padded rows and slices for a, b and dst; b and a 4-byte (not 16-byte)
    aligned; a stride-0 broadcast of a's slices."""
    rng = np.random.default_rng(21)
    for a_type, ne00 in ((synth.F32, 12), (synth.F32, 150), (synth.Q8_0, 64), (synth.Q4_K, 256)):
        K, ne02, ne10, ne12 = 37, 2, 70, 4
        if a_type == synth.F32:
            row = 4 * ne00 + 4 * 5                    # 5 floats of padding
        else:
            row = synth.row_bytes(a_type, ne00) + 8
        nb_a = [synth.BLOCK_BYTES[a_type], row, row * K + 12, 0]
        abytes = 4 + row * K * ne02 + 12 * ne02 + 64
        a = np.zeros(abytes, dtype=np.uint8)
        for s in range(ne02):
            for k in range(K):
                off = 4 + s * nb_a[2] + k * row
                if a_type == synth.F32:
                    a[off:off + 4 * ne00] = rng.standard_normal(ne00).astype(np.float32).view(np.uint8)
                else:
                    a[off:off + synth.row_bytes(a_type, ne00)] = synth.quant_rows(rng, a_type, 1, ne00)[0]
        a = a[4:]
        nb_b = [4, 4 * ne10 + 8, (4 * ne10 + 8) * K + 4, 0]
        b = np.zeros((nb_b[2] * ne12 + 16) // 4 + 1, dtype=np.float32)
        b[:] = rng.standard_normal(b.size).astype(np.float32)
        nb_d = [4, 4 * ne00 + 12, (4 * ne00 + 12) * ne10 + 4, 0]
        ne = [ne00, K, ne02, 1, ne10, K, ne12, 1, ne00, ne10, ne12, 1]
        nb = nb_a + nb_b + nb_d
        # device bases 4 bytes past a 256-byte boundary: no 16-byte vector loads
        gpu = G.run(a, a_type, b, ne, nb, a_off=4, b_off=4)
        ref, den = oracle.out_prod(a, a_type, b, ne, nb)
        res = oracle.check(gpu, ref, den, TOL)
        G.log("strided", synth.TYPE_NAMES[a_type], ne00, res)
        assert res["ok"], res
    # stride-0 broadcast of a over ne02
    inst = synth.make_instance("s0", synth.F32, (40, 50, 1, 1), (60, 50, 3, 1), 5)
    ne = list(inst.ne)
    nb = list(inst.nb)
    ne[2], nb[2] = 3, 0
    gpu = G.run(inst.a, synth.F32, inst.b, ne, nb)
    ref, den = oracle.out_prod(inst.a, synth.F32, inst.b, ne, nb)
    assert oracle.check(gpu, ref, den, TOL)["ok"]


def test_zero_K_and_empty_and_errors():
    ne, nb = synth.make_ne_nb(synth.F32, (8, 0, 1, 1), (100, 0, 1, 1))
    out = torch.full((100, 8), float("nan"), device="cuda:0")
    B.out_prod(0, synth.F32, 0, out.data_ptr(), ne, nb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (out == 0).all()
    # empty dst: nothing happens
    ne, nb = synth.make_ne_nb(synth.F32, (8, 10, 1, 1), (0, 10, 1, 1))
    B.out_prod(0, synth.F32, 0, 0, ne, nb, 0)
    # an error leaves dst untouched
    inst = synth.workload("lora_r8_single")
    a_d, b_d = G.to_dev(inst.a), G.to_dev(inst.b)
    out = torch.full((2560, 8), 7.0, device="cuda:0")
    ne = list(inst.ne)
    ne[5] = 511
    st = B.out_prod_status(a_d.data_ptr(), synth.F32, b_d.data_ptr(), out.data_ptr(), ne, inst.nb,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert B.STATUS[st] == "E_K" and (out == 7.0).all()


def test_tensor_helper_matches_raw_call():
    inst = synth.workload("deltanet_bcast")
    a_d, b_d = G.to_dev(inst.a), G.to_dev(inst.b)
    out = B.out_prod_tensors(a_d, synth.F32, b_d)
    torch.cuda.synchronize()
    raw = G.run(inst.a, inst.a_type, inst.b, inst.ne, inst.nb)
    assert np.array_equal(out.cpu().numpy(), raw)


def test_graph_capture_replays_match_eager():
    """Launches captured in a HIP graph: every replay, with eager work on the
    same buffers between replays, equals the eager result (b scaled by 2 in
    place between replays scales dst by exactly 2).  One uncaptured call on
    the capture stream first binds its workspace, so a plan that splits K
    (the rank-8 gradient) keeps its split under capture."""
    for name in ("lora_r8_single", "deltanet_bcast", "q8_0_5120"):
        inst = synth.workload(name)
        a_d = G.to_dev(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1))
        b_d = G.to_dev(inst.b)
        eager = torch.empty(inst.dst_shape, dtype=torch.float32, device="cuda:0")
        out = torch.empty_like(eager)
        stream = torch.cuda.current_stream().cuda_stream
        B.out_prod(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), eager.data_ptr(), inst.ne, inst.nb, stream)
        torch.cuda.synchronize()
        ref = eager.cpu().numpy()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        B.out_prod(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), out.data_ptr(), inst.ne, inst.nb,
                   cap.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            B.out_prod(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), out.data_ptr(), inst.ne, inst.nb,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        scale = 1.0
        for rep in range(4):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert np.array_equal(got, ref * np.float32(scale)), (name, rep)
            b_d.mul_(2.0)          # eager work on the captured buffer
            scale *= 2.0
        del g
        torch.cuda.synchronize()
        B.out_prod_release_stream(cap.cuda_stream)


# ---------------------------------------------------------------- b as a transposed view

KT_CASES = [
    (synth.F32, (8, 517, 1, 1), (333, 517, 1, 1)),
    (synth.F32, (4, 64, 1, 1), (100, 64, 1, 1)),       # K % 16 == 0: vector path
    (synth.F32, (24, 130, 2, 1), (70, 130, 4, 1)),
    (synth.F32, (300, 45, 2, 1), (290, 45, 4, 1)),
    (synth.Q8_0, (352, 70, 1, 1), (150, 70, 1, 1)),
    (synth.Q4_K, (768, 37, 1, 2), (141, 37, 1, 2)),
    (synth.Q4_K, (512, 64, 1, 1), (130, 64, 1, 1)),
]


@pytest.mark.parametrize("a_type,a_ne,b_ne", KT_CASES)
def test_k_contiguous_b(a_type, a_ne, b_ne):
    """b stored K-contiguous (the grad^T view of the matmul backward)."""
    inst = synth.make_instance("kt", a_type, a_ne, b_ne, seed_of("kt", a_ne, b_ne), b_kt=True)
    assert inst.b_kt
    check_case(inst)


@pytest.mark.parametrize("cfg", B.TILED_CONFIGS)
def test_k_contiguous_b_every_tiled_configuration(cfg):
    code = B.kernel_code(B.KERNEL_TILED, cfg)
    for a_type, a_ne, b_ne in KT_CASES[3:]:
        inst = synth.make_instance("ktcfg", a_type, a_ne, b_ne, seed_of("ktc", cfg, a_ne), b_kt=True)
        check_case(inst, code)


@pytest.mark.parametrize("cfg", [0, 5, 6])
def test_k_contiguous_b_column_configurations(cfg):
    code = B.kernel_code(B.KERNEL_SKINNY, cfg)
    for a_type, a_ne, b_ne in KT_CASES[:4]:
        inst = synth.make_instance("ktcol", a_type, a_ne, b_ne, seed_of("ktcol", cfg, a_ne), b_kt=True)
        check_case(inst, code)
    # misaligned b: scalar loads
    inst = synth.make_instance("ktmis", synth.F32, (8, 64, 1, 1), (40, 64, 1, 1), cfg, b_kt=True)
    gpu = G.run(inst.a, synth.F32, inst.b, inst.ne, inst.nb, code, b_off=4)
    ref, den = oracle.out_prod(inst.a, synth.F32, inst.b, inst.ne, inst.nb)
    assert oracle.check(gpu, ref, den, TOL)["ok"]


@pytest.mark.parametrize("name", ["q4_K_5120x17408", "q4_K_17408x5120", "q8_0_5120", "lora_r8_9216"])
def test_k_contiguous_b_full_size(name):
    """Input gradient through a frozen weight, out_prod(W, grad^T), at full size."""
    a_type, a_ne, b_ne, seed, a_std, b_kind = synth.WORKLOADS[name][:6]
    inst = synth.make_instance(name + "_kt", a_type, a_ne, b_ne, seed, a_std, b_kind, b_kt=True)
    n = b_ne[0]
    cols = None
    if inst.ne[0] * inst.ne[1] * n > 5e9:
        cols = np.array([[i1, 0, 0] for i1 in (0, 1, n // 3, n - 1)])
    check_case(inst, 0, cols)


# ---------------------------------------------------------------- narrow b (operand swap)

@pytest.mark.parametrize("a_ne,b_ne", [
    ((2560, 512, 1, 1), (8, 512, 1, 1)),     # LoRA down-projection gradient out_prod(x, grad_h)
    ((300, 77, 2, 1), (8, 77, 4, 1)),        # broadcast on the wide operand
    ((130, 33, 1, 3), (24, 33, 2, 3)),
    ((40, 5, 1, 1), (1, 5, 1, 1)),
])
def test_narrow_b_operand_swap(a_ne, b_ne):
    inst = synth.make_instance("nb", synth.F32, a_ne, b_ne, seed_of("nb", a_ne))
    p = B.out_prod_plan(0x10000000, synth.F32, 0x40000000000, 0x80000000000, inst.ne, inst.nb)
    assert p["swapped"] == 1
    check_case(inst)
    # dst with padded rows (the swapped store walks dst's strides)
    nb = list(inst.nb)
    nb[9] = 4 * a_ne[0] + 20
    nb[10] = nb[9] * b_ne[0] + 8
    nb[11] = nb[10] * b_ne[2]
    gpu = G.run(inst.a, synth.F32, inst.b, inst.ne, nb)
    ref, den = oracle.out_prod(inst.a, synth.F32, inst.b, inst.ne, nb)
    assert oracle.check(gpu, ref, den, TOL)["ok"]


# ---------------------------------------------------------------- split K

SPLIT_CASES = [
    # (a_type, a_ne, b_ne, K-contiguous b, family, configuration or None, splits)
    (synth.F32, (40, 300, 1, 1), (70, 300, 1, 1), False, B.KERNEL_TILED, None, 3),
    # 61-row ranges: K-contiguous b loses 16-byte alignment past range 0
    (synth.F32, (40, 301, 2, 1), (70, 301, 4, 1), True, B.KERNEL_TILED, None, 5),
    (synth.F32, (130, 97, 1, 1), (129, 97, 1, 1), False, B.KERNEL_TILED, 1, 2),
    (synth.F32, (8, 517, 1, 1), (333, 517, 1, 1), False, B.KERNEL_SKINNY, None, 4),
    (synth.F32, (8, 517, 1, 1), (333, 517, 1, 1), True, B.KERNEL_SKINNY, None, 7),
    (synth.F32, (24, 130, 2, 1), (70, 130, 4, 1), True, B.KERNEL_SKINNY, None, 2),
    (synth.F32, (3, 200, 1, 2), (50, 200, 1, 2), False, B.KERNEL_SKINNY, 6, 6),
    (synth.F32, (8, 300, 1, 1), (200, 300, 1, 1), False, B.KERNEL_SKINNY, 10, 3),
    (synth.F32, (33, 150, 1, 1), (90, 150, 1, 1), False, B.KERNEL_SKINNY, 3, 5),
    (synth.Q8_0, (352, 70, 1, 1), (150, 70, 1, 1), False, B.KERNEL_TILED, None, 2),
    (synth.Q4_K, (768, 37, 1, 2), (141, 37, 1, 2), True, B.KERNEL_TILED, None, 3),
    (synth.Q4_K, (512, 200, 1, 1), (130, 200, 1, 1), False, B.KERNEL_TILED, None, 64),
]


@pytest.mark.parametrize("a_type,a_ne,b_ne,kt,fam,cfg,splits", SPLIT_CASES)
def test_split_k_forced(a_type, a_ne, b_ne, kt, fam, cfg, splits):
    """K split into ranges whose partials the reduce kernel adds: parity with
    the oracle, and two runs are bit-identical."""
    inst = synth.make_instance("split", a_type, a_ne, b_ne, seed_of("split", a_ne, b_ne, kt), b_kt=kt)
    code = B.kernel_code(fam, cfg, splits)
    p = B.out_prod_plan(0x10000000, a_type, 0x40000000000, 0x80000000000, inst.ne, inst.nb, code)
    assert p["splits"] > 1
    gpu = check_case(inst, code)
    again = G.run(inst.a, a_type, inst.b, inst.ne, inst.nb, code)
    assert np.array_equal(gpu, again)


def test_split_k_integer_exact_equals_unsplit():
    """Integer data: every summation order is exact, so the split result equals
    the unsplit one and the exact sum bit for bit."""
    rng = np.random.default_rng(seed_of("split-int"))
    for kt, fam in ((False, B.KERNEL_TILED), (True, B.KERNEL_TILED), (False, B.KERNEL_SKINNY),
                    (True, B.KERNEL_SKINNY)):
        M = 40 if fam == B.KERNEL_TILED else 8
        inst = synth.make_instance("si", synth.F32, (M, 777, 1, 1), (90, 777, 1, 1), 5, b_kt=kt)
        a = _int_f32(rng, inst.a.shape)
        b = _int_f32(rng, (777, 90))
        b_host = np.ascontiguousarray(b.T) if kt else b
        exact = (b.astype(np.float64).T @ a[0, 0].astype(np.float64)).astype(np.float32)
        one = G.run(a, synth.F32, b_host, inst.ne, inst.nb, B.kernel_code(fam, None, 1))
        many = G.run(a, synth.F32, b_host, inst.ne, inst.nb, B.kernel_code(fam, None, 9))
        assert np.array_equal(one[0, 0], exact) and np.array_equal(many[0, 0], exact)


def test_split_k_operand_swapped_auto():
    """A narrow f32 b with a long K: the operand-swapped column launch splits K,
    and the reduce writes dst through the exchanged strides (padded rows too)."""
    inst = synth.make_instance("nbs", synth.F32, (300, 2048, 1, 1), (8, 2048, 1, 1), seed_of("nbs"))
    p = B.out_prod_plan(0x10000000, synth.F32, 0x40000000000, 0x80000000000, inst.ne, inst.nb)
    assert p["swapped"] == 1 and p["splits"] > 1
    check_case(inst)
    nb = list(inst.nb)
    nb[9] = 4 * 300 + 20
    nb[10] = nb[9] * 8
    nb[11] = nb[10]
    gpu = G.run(inst.a, synth.F32, inst.b, inst.ne, nb)
    ref, den = oracle.out_prod(inst.a, synth.F32, inst.b, inst.ne, nb)
    assert oracle.check(gpu, ref, den, TOL)["ok"]


# ---------------------------------------------------------------- every a type

NEW_TYPES = [synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0, synth.Q5_1,
             synth.Q2_K, synth.Q3_K, synth.Q5_K, synth.Q6_K]
ALL_TYPES = [synth.F32, synth.Q8_0, synth.Q4_K] + NEW_TYPES


def _type_shapes(a_type):
    """Shapes spanning several tiles with a ragged tail and a broadcast slice
    dim: (a_ne, b_ne) pairs."""
    qk = synth.BLOCK_VALUES[a_type]
    if qk == 1:
        return [((203, 45, 2, 1), (77, 45, 4, 1)), ((300, 130, 1, 1), (290, 130, 1, 1)),
                ((16, 9, 1, 1), (5, 9, 1, 1))]
    if qk == 32:
        return [((160, 33, 2, 1), (130, 33, 4, 1)), ((352, 70, 1, 1), (150, 70, 1, 1)),
                ((32, 1, 1, 1), (7, 1, 1, 1))]
    return [((768, 37, 1, 2), (141, 37, 1, 2)), ((512, 64, 1, 1), (130, 64, 1, 1)),
            ((256, 1, 1, 1), (5, 1, 1, 1))]


@pytest.mark.parametrize("a_type", ALL_TYPES)
def test_every_type_small_ragged(a_type):
    """Each a type: ragged and broadcast shapes, b row-major and K-contiguous,
    unsplit and split K, and a 2-byte offset a where the type allows it."""
    for i, (a_ne, b_ne) in enumerate(_type_shapes(a_type)):
        for kt in (False, True):
            inst = synth.make_instance("t%d" % a_type, a_type, a_ne, b_ne,
                                       seed_of("types", a_type, i, kt), b_kt=kt)
            check_case(inst, B.kernel_code(B.KERNEL_TILED) if a_type == synth.F32 else 0)
            if a_ne[1] >= 4:
                check_case(inst, B.kernel_code(B.KERNEL_TILED, None, 3))
    if synth.BLOCK_BYTES[a_type] % 4 != 0:
        a_ne, b_ne = _type_shapes(a_type)[0]
        inst = synth.make_instance("off", a_type, a_ne, b_ne, seed_of("off", a_type))
        gpu = G.run(inst.a, a_type, inst.b, inst.ne, inst.nb, a_off=2)
        ref, den = oracle.out_prod(inst.a, a_type, inst.b, inst.ne, inst.nb)
        assert oracle.check(gpu, ref, den, TOL)["ok"]


def _integer_a(rng, a_type, nrows, ne00):
    """a whose decoded values are integers: fp16 scales 1, q4_1/q5_1 offsets
    -8; f16 / bf16 integer values in [-8, 8]."""
    if a_type in (synth.F16, synth.BF16):
        x = rng.integers(-8, 9, size=(nrows, ne00)).astype(np.float32)
        return x.astype(np.float16).view(np.uint16) if a_type == synth.F16 else \
            (x.view(np.uint32) >> 16).astype(np.uint16)
    if a_type == synth.F32:
        return rng.integers(-8, 9, size=(nrows, ne00)).astype(np.float32)
    one = int(synth.fp16_bits([1.0])[0])
    minus8 = int(synth.fp16_bits([-8.0])[0])
    if a_type == synth.Q8_0:
        return synth.q8_0_rows(rng, nrows, ne00, d_bits=one)
    if a_type == synth.Q4_K:
        return synth.q4_K_rows(rng, nrows, ne00, d_bits=one, dmin_bits=one)
    return synth.block_rows(rng, a_type, nrows, ne00, half_bits={"scale": one, "offset": minus8})


@pytest.mark.parametrize("a_type", ALL_TYPES)
def test_every_type_integer_exact(a_type):
    """Integer-valued a (unit fp16 scales) and b in {-1, 0, 1}: every partial
    sum is an integer below 2^24 (|value| <= 4096 for q6_K, K = 2048), so
    the whole dst equals the oracle bit for bit, row-major and K-contiguous b."""
    M, K, N = 2560, 2048, 512
    rng = synth.rng_for(seed_of("int-type", a_type))
    a = _integer_a(rng, a_type, K, M).reshape(1, 1, K, -1)
    b = rng.integers(-1, 2, size=(1, 1, K, N)).astype(np.float32)
    for kt in (False, True):
        ne, nb = synth.make_ne_nb(a_type, (M, K, 1, 1), (N, K, 1, 1), b_kt=kt)
        bh = np.ascontiguousarray(b.transpose(0, 1, 3, 2)) if kt else b
        G.log("int-exact", synth.TYPE_NAMES[a_type], "kt", kt)
        gpu = G.run(a, a_type, bh, ne, nb)
        ref, _ = oracle.out_prod(a, a_type, bh, ne, nb)
        assert np.array_equal(gpu, ref.astype(np.float32))


@pytest.mark.parametrize("a_type", NEW_TYPES)
def test_every_type_dequant_bit_exact_one_hot(a_type):
    """One-hot b copies row k of a into dst column i1: dst holds the kernel's
    own decoded values, which must equal the oracle's decode bit for bit (as
    values) for every row of a 2560 x 1024 weight."""
    M, K, N = 2560, 1024, 512
    inst = synth.make_instance("oh", a_type, (M, K, 1, 1), (N, K, 1, 1), seed_of("onehot", a_type))
    rowb = inst.a.shape[-1] * inst.a.itemsize
    raw = np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1)
    expect = oracle.dequant_rows(raw, a_type, M, K, rowb)
    a_d = G.to_dev(raw)
    out = torch.empty((N, M), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for start in range(0, K, N):
        rows = np.arange(start, min(K, start + N))
        b_d = torch.zeros((K, N), dtype=torch.float32, device="cuda:0")
        b_d[torch.from_numpy(rows).to("cuda:0"), torch.arange(rows.size, device="cuda:0")] = 1.0
        out.fill_(float("nan"))
        B.out_prod(a_d.data_ptr(), a_type, b_d.data_ptr(), out.data_ptr(), inst.ne, inst.nb, stream)
        got = out[: rows.size].cpu().numpy()
        assert np.array_equal(got, expect[rows]), (synth.TYPE_NAMES[a_type], start)


@pytest.mark.parametrize("a_type", [synth.Q8_0, synth.Q4_K, synth.Q2_K, synth.Q6_K, synth.Q4_1, synth.F16])
def test_subnormal_half_scales_bit_exact(a_type):
    """fp16 scales (and f16 weights) that are subnormal, zero or negative decode
    exactly: one-hot b reads the kernel's decoded values back, compared bit for
    bit (as values) with the oracle's decode.  Pins the half -> float
    conversion, subnormals included."""
    M, K, N = 512, 64, 64
    rng = synth.rng_for(seed_of("subn", a_type))
    if a_type == synth.F16:
        bits = rng.integers(0, 0x7C00, size=(K, M)).astype(np.uint16)      # finite, incl. subnormal
        bits[:, ::3] = rng.integers(0, 0x0400, size=bits[:, ::3].shape)     # a third subnormal
        bits |= (rng.integers(0, 2, size=bits.shape) << 15).astype(np.uint16)
        a = bits
    else:
        a = synth.quant_rows(rng, a_type, K, M) if a_type in (synth.Q8_0, synth.Q4_K) else \
            synth.block_rows(rng, a_type, K, M)
        qk, bb = synth.BLOCK_VALUES[a_type], synth.BLOCK_BYTES[a_type]
        blocks = a.reshape(K, M // qk, bb)
        for off, _ in synth.HALF_FIELDS[a_type]:
            h = rng.integers(0, 0x0400, size=blocks.shape[:2]).astype(np.uint16)   # subnormal or 0
            h |= (rng.integers(0, 2, size=h.shape) << 15).astype(np.uint16)
            blocks[:, :, off:off + 2] = h.reshape(K, -1, 1).view(np.uint8).reshape(K, -1, 2)
        a = blocks.reshape(K, -1)
    raw = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    rowb = raw.size // K
    expect = oracle.dequant_rows(raw, a_type, M, K, rowb)
    ne, nb = synth.make_ne_nb(a_type, (M, K, 1, 1), (N, K, 1, 1))
    b = np.eye(K, N, dtype=np.float32)        # column i1 picks row k = i1 of a
    gpu = G.run(raw, a_type, b, ne, nb)
    assert np.array_equal(gpu[0, 0], expect[:N])
