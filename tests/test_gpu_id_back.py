"""Parity of the HIP MUL_MAT_ID_BACK path (through the C ABI) with the CPU oracle.

Gate as for OUT_PROD: no NaN/Inf except where an id is not an expert (that row
must be all NaN), |gpu - ref| <= 1e-5 * sum_r |a||g| per element.  Routing is
seeded: distinct top-k experts per token, plus skewed and invalid routings.
"""
import dataclasses
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
ALL_TYPES = [synth.F32, synth.F16, synth.BF16, synth.Q4_0, synth.Q4_1, synth.Q5_0, synth.Q5_1,
             synth.Q8_0, synth.Q2_K, synth.Q3_K, synth.Q4_K, synth.Q5_K, synth.Q6_K]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield


def seed_of(*parts):
    return zlib.crc32(repr(parts).encode()) & 0x7FFFFFFF


def run_id(inst, ids=None, kernel=0, nb=None, stream=None):
    """MUL_MAT_ID_BACK on cuda:0; returns dst as (n_tokens, n_used, ne00) through
    dst's strides (nb may pad g and dst)."""
    ids = inst.ids if ids is None else ids
    ne = inst.ne
    nb = list(inst.nb) if nb is None else list(nb)
    ne00, n_used, n_tok = ne[12], ne[13], ne[14]
    a_d = G.to_dev(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1))
    # g through its strides
    g_floats = max(1, (ne[4] - 1) + (n_used - 1) * nb[5] // 4 + (n_tok - 1) * nb[6] // 4 + 1)
    g_host = np.zeros(g_floats, dtype=np.float32)
    for t in range(n_tok):
        for i in range(n_used):
            o = (i * nb[5] + t * nb[6]) // 4
            g_host[o:o + ne[4]] = inst.g[t, i]
    g_d = G.to_dev(g_host)
    i_d = G.to_dev(np.ascontiguousarray(ids, dtype=np.int32))
    d_floats = max(1, (ne00 - 1) + (n_used - 1) * nb[13] // 4 + (n_tok - 1) * nb[14] // 4 + 1)
    d_d = torch.full((d_floats,), 12345.0, dtype=torch.float32, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    st = B.out_prod_id_back_status(a_d.data_ptr(), inst.a_type, g_d.data_ptr(), i_d.data_ptr(),
                                   d_d.data_ptr(), ne, nb, s, kernel)
    assert st == 0, B.STATUS.get(st)
    torch.cuda.synchronize()
    flat = d_d.cpu().numpy()
    out = np.empty((n_tok, n_used, ne00), dtype=np.float32)
    for t in range(n_tok):
        for i in range(n_used):
            o = (i * nb[13] + t * nb[14]) // 4
            out[t, i] = flat[o:o + ne00]
    return out, flat


def check_id(inst, gpu, slots=None, nb=None):
    nb = inst.nb if nb is None else nb
    ref, den = oracle.mul_mat_id_back(inst.a, inst.a_type, inst.g, inst.ids, inst.ne, inst.nb,
                                      slots=slots)
    if slots is None:
        res = oracle.check(gpu, ref, den, TOL)
    else:
        n_used = inst.ne[5]
        g = np.stack([gpu[s // n_used, s % n_used] for s in slots])
        res = oracle.check(g, ref, den, TOL)
    G.log("   ", res)
    assert res["ok"], res


def _shape(a_type):
    qk = synth.BLOCK_VALUES[a_type]
    return (200 if qk == 1 else 96 if qk == 32 else 512), 77


@pytest.mark.parametrize("a_type", ALL_TYPES)
def test_id_back_every_type(a_type):
    """Each expert type, ragged K, 6 experts (some with several tiles of slots,
    some with none), 3 used of 6 per token."""
    ne00, K = _shape(a_type)
    inst = synth.make_moe_instance("t", a_type, ne00, K, 6, 3, 70, seed_of("idt", a_type))
    G.log("case id_back", synth.TYPE_NAMES[a_type], inst.ne[:3], "slots", 210)
    gpu, _ = run_id(inst)
    check_id(inst, gpu)


@pytest.mark.parametrize("cfg", B.ID_CONFIGS)
def test_id_back_every_configuration(cfg):
    inst = synth.make_moe_instance("c", synth.Q4_K, 768, 130, 9, 4, 150, seed_of("idc", cfg))
    gpu, _ = run_id(inst, kernel=B.kernel_code(B.KERNEL_TILED, cfg))
    check_id(inst, gpu)


@pytest.mark.parametrize("a_type", ALL_TYPES)
def test_id_back_whole_stages_every_type(a_type):
    """K a whole number of 32-row stages and ne00 = 512 (whole m-tiles for
    most tile heights), partly filled slot tiles."""
    inst = synth.make_moe_instance("tp", a_type, 512, 128, 6, 3, 70, seed_of("idtp", a_type))
    G.log("case id_back whole stages", synth.TYPE_NAMES[a_type], inst.ne[:3], "slots", 210)
    gpu, _ = run_id(inst)
    check_id(inst, gpu)


@pytest.mark.parametrize("cfg", B.ID_CONFIGS)
@pytest.mark.parametrize("shape", [(768, 160, 9, 4, 150), (1024, 256, 5, 4, 150)])
def test_id_back_whole_stages_every_configuration(cfg, shape):
    """Whole stages and aligned columns (and, where 768 is not a multiple of
    the tile height, a ragged last m-tile); 5 experts of 120 slots on average
    give full slot tiles (the unchecked loop) next to partly filled ones."""
    ne00, K, n_e, n_u, n_t = shape
    inst = synth.make_moe_instance("cp", synth.Q4_K, ne00, K, n_e, n_u, n_t, seed_of("idcp", cfg, ne00))
    G.log("case id_back whole stages cfg", cfg, inst.ne[:3])
    gpu, _ = run_id(inst, kernel=B.kernel_code(B.KERNEL_TILED, cfg))
    check_id(inst, gpu)


def test_id_back_skewed_routing_and_repeat():
    """Every slot routed to one expert (many tiles of one expert), then a
    routing that leaves most experts empty; two runs are bit-identical."""
    inst = synth.make_moe_instance("sk", synth.Q8_0, 160, 64, 12, 1, 600, seed_of("sk"))
    inst.ids[:] = 7
    gpu, _ = run_id(inst)
    check_id(inst, gpu)
    again, _ = run_id(inst)
    assert np.array_equal(gpu.view(np.uint32), again.view(np.uint32))
    inst.ids[:] = np.where(np.arange(600)[:, None] % 3 == 0, 11, 2).astype(np.int32)
    gpu, _ = run_id(inst)
    check_id(inst, gpu)


def test_id_back_routing_paths_agree():
    """18000 slots (past the one-block routing kernel's 16384: the three
    routing kernels), with three invalid ids, against the oracle; the first
    2000 tokens alone (12000 slots, one-block routing) give bit-identical
    rows."""
    inst = synth.make_moe_instance("many", synth.Q8_0, 64, 32, 40, 6, 3000, seed_of("many"))
    ids = inst.ids.copy()
    bad = [(5, 2, 40), (1999, 0, -3), (2999, 5, 1 << 30)]
    for t, i, v in bad:
        ids[t, i] = v
    gpu, _ = run_id(inst, ids=ids)
    valid = np.ones((3000, 6), dtype=bool)
    for t, i, _ in bad:
        valid[t, i] = False
        assert np.isnan(gpu[t, i]).all()
    slots = [t * 6 + i for t in range(3000) for i in range(6) if valid[t, i]]
    ref = dataclasses.replace(inst, ids=np.where(valid, ids, 0).astype(np.int32))
    check_id(ref, gpu, slots=slots)         # oracle: the valid slots only
    ne = list(inst.ne)
    ne[6] = ne[9] = ne[14] = 2000           # g, ids and dst over the first 2000 tokens
    small, _ = run_id(dataclasses.replace(inst, ne=ne), ids=ids)
    assert np.array_equal(small.view(np.uint32), gpu[:2000].view(np.uint32))


@pytest.mark.parametrize("n_tok", [8192, 8193])
def test_id_back_routing_limit(n_tok):
    """2 slots per token: 16384 slots (the most the one-block routing takes)
    and 16386 (the three routing kernels), against the oracle."""
    inst = synth.make_moe_instance("lim", synth.Q4_0, 64, 16, 12, 2, n_tok, seed_of("lim", n_tok))
    G.log("case id_back routing limit", n_tok * 2, "slots")
    gpu, _ = run_id(inst)
    check_id(inst, gpu)


def test_id_back_invalid_ids_give_nan_rows():
    inst = synth.make_moe_instance("bad", synth.F32, 64, 40, 5, 2, 30, seed_of("bad"))
    ids = inst.ids.copy()
    bad = [(3, 1, 5), (10, 0, -1), (29, 1, 1 << 20)]
    for t, i, v in bad:
        ids[t, i] = v
    gpu, _ = run_id(inst, ids=ids)
    valid = np.ones((30, 2), dtype=bool)
    for t, i, _ in bad:
        valid[t, i] = False
        assert np.isnan(gpu[t, i]).all()
    slots = [t * 2 + i for t in range(30) for i in range(2) if valid[t, i]]
    inst.ids = np.where(valid, ids, 0).astype(np.int32)   # oracle: the valid slots only
    check_id(inst, gpu, slots=slots)


def test_id_back_strided_g_and_dst_and_zero_k():
    inst = synth.make_moe_instance("st", synth.Q5_K, 256, 50, 4, 2, 9, seed_of("st"))
    nb = list(inst.nb)
    nb[5] = 4 * 50 + 12          # padded g rows (not 16-byte aligned: scalar path)
    nb[6] = nb[5] * 2 + 36
    nb[13] = 4 * 256 + 20        # padded dst rows
    nb[14] = nb[13] * 2 + 8
    gpu, flat = run_id(inst, nb=nb)
    check_id(inst, gpu)
    # padding between dst rows untouched
    assert flat[256] == 12345.0
    # K == 0: zeros, ids not read
    z = synth.make_moe_instance("z", synth.F32, 32, 0, 3, 2, 4, 1)
    out, _ = run_id(z, ids=np.full((4, 2), -5, dtype=np.int32))
    assert not out.any()


def test_id_back_graph_capture_replays():
    """Captured after one uncaptured call on the capture stream (the routing
    tables live in that stream's workspace): every replay equals eager, with
    eager writes to the captured buffers between replays."""
    inst = synth.make_moe_instance("gr", synth.Q4_K, 512, 96, 8, 2, 100, seed_of("gr"))
    eager, _ = run_id(inst)
    a_d = G.to_dev(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1))
    g_d = G.to_dev(inst.g)
    i_d = G.to_dev(inst.ids)
    out = torch.zeros(inst.dst_shape, dtype=torch.float32, device="cuda:0")
    args = (a_d.data_ptr(), inst.a_type, g_d.data_ptr(), i_d.data_ptr(), out.data_ptr(), inst.ne, inst.nb)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    B.out_prod_id_back(*args, cap.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        B.out_prod_id_back(*args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    scale = 1.0
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager * np.float32(scale)), rep
        g_d.mul_(2.0)
        scale *= 2.0


@pytest.mark.parametrize("name", list(synth.MOE_WORKLOADS))
def test_id_back_full_size(name):
    """The bench's MoE shapes (64 q4_K experts, 8 of 64 routed, 512 tokens),
    oracle on sampled slots."""
    inst = synth.moe_workload(name)
    G.log("case", name, inst.ne[:7])
    gpu, _ = run_id(inst)
    assert np.isfinite(gpu).all()
    rng = np.random.default_rng(seed_of("full", name))
    n = inst.ne[5] * inst.ne[6]
    slots = sorted(set([0, n - 1] + list(rng.choice(n, 40, replace=False))))
    check_id(inst, gpu, slots=slots)
