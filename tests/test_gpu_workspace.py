"""The library's workspace pool on the GPU (split-K partials, MUL_MAT_ID_BACK
routing tables): at most 4 workspaces per device, each bound to one stream,
freed by out_prod_release_stream; a splitting out_prod without a workspace
runs unsplit; graph capture on a stream with and without one.

Every call goes through the C ABI on raw HIP streams; results are checked
against the CPU oracle with the parity gate, or bit for bit against the
eager result of the same plan."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TOL = 1e-5
POOL = 4
WS_BYTES = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.load_library()
    yield


def _hip():
    lib = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch already loaded
    lib.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return lib


class Streams:
    """Raw HIP streams, released from the pool and destroyed on exit."""

    def __init__(self):
        self.hip = _hip()
        self.live = []

    def new(self):
        raw = ctypes.c_void_p()
        assert self.hip.hipStreamCreate(ctypes.byref(raw)) == 0
        self.live.append(raw.value)
        return raw.value

    def close(self, s):
        B.out_prod_release_stream(s)
        assert self.hip.hipStreamDestroy(ctypes.c_void_p(s)) == 0
        self.live.remove(s)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        torch.cuda.synchronize()
        for s in list(self.live):
            self.close(s)


class Problem:
    """A workload's inputs on the device and a dst buffer."""

    def __init__(self, name):
        self.inst = synth.workload(name)
        i = self.inst
        self.a = G.to_dev(np.ascontiguousarray(i.a).view(np.uint8).reshape(-1))
        self.b = G.to_dev(i.b)
        self.out = torch.full(i.dst_shape, float("nan"), dtype=torch.float32, device="cuda:0")
        self.plan = B.out_prod_plan(self.a.data_ptr(), i.a_type, self.b.data_ptr(), self.out.data_ptr(),
                                    i.ne, i.nb)

    def call(self, stream, kernel=0):
        i = self.inst
        return B.out_prod_status(self.a.data_ptr(), i.a_type, self.b.data_ptr(), self.out.data_ptr(),
                                 i.ne, i.nb, stream, kernel)

    def result(self):
        torch.cuda.synchronize()
        return self.out.cpu().numpy()

    def check_oracle(self):
        i = self.inst
        ref, den = oracle.out_prod(i.a, i.a_type, i.b, i.ne, i.nb)
        res = oracle.check(self.result(), ref, den, TOL)
        assert res["ok"], res


def _release_all_known(streams):
    for s in streams:
        B.out_prod_release_stream(s)


def test_stream_cycling_keeps_the_pool_bounded():
    """16 streams, created and destroyed one after another, each making one
    splitting call: every call returns the same bits, the pool never holds
    more than one workspace here, and the device's free memory ends within
    one pool (4 x 64 MiB) of where it started."""
    dh = Problem("lora4B_dh")
    assert dh.plan["splits"] > 1
    cur = torch.cuda.current_stream().cuda_stream
    B.out_prod_release_stream(cur)
    assert dh.call(cur) == 0
    ref = dh.result()
    B.out_prod_release_stream(cur)
    torch.cuda.synchronize()
    n0 = B.out_prod_workspace_count()
    free0 = torch.cuda.mem_get_info()[0]
    with Streams() as st:
        for k in range(16):
            s = st.new()
            dh.out.fill_(float("nan"))
            torch.cuda.synchronize()
            assert dh.call(s) == 0
            assert np.array_equal(dh.result(), ref), k
            assert B.out_prod_workspace_count() == n0 + 1
            st.close(s)
            assert B.out_prod_workspace_count() == n0
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    G.log("free memory before/after 16 streams (MiB):", free0 >> 20, free1 >> 20, "pool", n0)
    assert free1 >= free0 - POOL * WS_BYTES


def test_pool_cap_and_fallback():
    """With 4 streams holding workspaces, a fifth stream's splitting out_prod
    runs unsplit (parity with the oracle), a forced split and MUL_MAT_ID_BACK
    are refused with E_WORKSPACE (dst untouched), and releasing one stream
    lets the fifth bind a workspace and split again."""
    dh = Problem("lora4B_dh")
    cur = torch.cuda.current_stream().cuda_stream
    B.out_prod_release_stream(cur)
    moe = synth.make_moe_instance("ws_moe", synth.Q4_K, 256, 64, 8, 2, 40, 7)
    ma = G.to_dev(np.ascontiguousarray(moe.a).view(np.uint8).reshape(-1))
    mg = G.to_dev(moe.g)
    mi = G.to_dev(moe.ids)
    md = torch.full(moe.dst_shape, 7.0, dtype=torch.float32, device="cuda:0")
    forced = B.kernel_code(B.KERNEL_SKINNY, dh.plan["variant"], dh.plan["splits"])
    with Streams() as st:
        n0 = B.out_prod_workspace_count()
        assert n0 < POOL, "other streams of this process hold every workspace"
        holders = [st.new() for _ in range(POOL - n0)]
        for s in holders:
            assert dh.call(s) == 0
        torch.cuda.synchronize()
        assert B.out_prod_workspace_count() == POOL
        split_bits = dh.result()
        fifth = st.new()
        dh.out.fill_(float("nan"))
        torch.cuda.synchronize()
        assert dh.call(fifth) == 0          # unsplit fallback
        dh.check_oracle()
        assert B.out_prod_workspace_count() == POOL
        dh.out.fill_(3.0)
        torch.cuda.synchronize()
        assert B.STATUS[dh.call(fifth, forced)] == "E_WORKSPACE"
        assert (dh.result() == 3.0).all()
        st_id = B.out_prod_id_back_status(ma.data_ptr(), moe.a_type, mg.data_ptr(), mi.data_ptr(),
                                          md.data_ptr(), moe.ne, moe.nb, fifth)
        assert B.STATUS[st_id] == "E_WORKSPACE"
        torch.cuda.synchronize()
        assert (md.cpu().numpy() == 7.0).all()
        st.close(holders[0])
        assert B.out_prod_workspace_count() == POOL - 1
        assert dh.call(fifth, forced) == 0
        assert np.array_equal(dh.result(), split_bits)
        assert B.out_prod_id_back_status(ma.data_ptr(), moe.a_type, mg.data_ptr(), mi.data_ptr(),
                                         md.data_ptr(), moe.ne, moe.nb, fifth) == 0
        torch.cuda.synchronize()
        ref, den = oracle.mul_mat_id_back(moe.a, moe.a_type, moe.g, moe.ids, moe.ne, moe.nb)
        got = md.cpu().numpy()
        assert oracle.check(got.reshape(ref.shape), ref, den, TOL)["ok"]
    assert B.out_prod_workspace_count() == n0


def test_split_k_in_graph_capture():
    """Capture on a stream that holds no workspace: a splitting out_prod is
    captured unsplit (every replay the same bits, within the gate), a forced
    split and MUL_MAT_ID_BACK are refused with E_CAPTURE and nothing is
    enqueued.  After one uncaptured call binds a workspace, the captured
    splitting call replays bit for bit equal to the eager result, with eager
    work on the captured buffers between replays."""
    cur = torch.cuda.current_stream().cuda_stream
    B.out_prod_release_stream(cur)
    n0 = B.out_prod_workspace_count()
    assert n0 < POOL, "other streams of this process hold every workspace"
    with Streams() as st:
        raw = st.new()
        ext = torch.cuda.ExternalStream(raw)
        for name in ("lora4B_dh", "lora4B_dxW"):
            pr = Problem(name)
            inst = pr.inst
            assert pr.plan["splits"] > 1
            eager = torch.empty(inst.dst_shape, dtype=torch.float32, device="cuda:0")
            B.out_prod(pr.a.data_ptr(), inst.a_type, pr.b.data_ptr(), eager.data_ptr(), inst.ne, inst.nb, cur)
            torch.cuda.synchronize()
            ref = eager.cpu().numpy()
            B.out_prod_release_stream(cur)
            if name == "lora4B_dh":
                assert B.out_prod_workspace_count() == n0
                fam = B.KERNEL_SKINNY
                forced = B.kernel_code(fam, pr.plan["variant"], pr.plan["splits"])
                g0 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g0, stream=ext):
                    pr.out.zero_()
                    st_forced = pr.call(raw, forced)
                    st_auto = pr.call(raw)
                assert B.STATUS[st_forced] == "E_CAPTURE"
                assert st_auto == 0
                assert B.out_prod_workspace_count() == n0
                torch.cuda.synchronize()
                first = None
                for rep in range(3):
                    pr.out.fill_(float("nan"))
                    torch.cuda.synchronize()
                    g0.replay()
                    got = pr.result()
                    if first is None:
                        first = got
                        pr.check_oracle()
                    assert np.array_equal(got, first), rep
                del g0
                torch.cuda.synchronize()
                ext.wait_stream(torch.cuda.current_stream())
                assert pr.call(raw) == 0    # uncaptured: binds the stream's workspace
                assert np.array_equal(pr.result(), ref)
                assert B.out_prod_workspace_count() == n0 + 1
            g = torch.cuda.CUDAGraph()
            ext.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(g, stream=ext):
                assert pr.call(raw) == 0
            torch.cuda.synchronize()
            scale = 1.0
            for rep in range(4):
                pr.out.fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                assert np.array_equal(pr.result(), ref * np.float32(scale)), (name, rep)
                pr.b.mul_(2.0)
                scale *= 2.0
            del g
            torch.cuda.synchronize()
        # MUL_MAT_ID_BACK under capture on a stream without a workspace
        st.close(raw)
        raw = st.new()
        ext = torch.cuda.ExternalStream(raw)
        moe = synth.make_moe_instance("cap_moe", synth.Q8_0, 64, 32, 4, 2, 16, 11)
        ma = G.to_dev(np.ascontiguousarray(moe.a).view(np.uint8).reshape(-1))
        mg, mi = G.to_dev(moe.g), G.to_dev(moe.ids)
        md = torch.zeros(moe.dst_shape, dtype=torch.float32, device="cuda:0")
        g1 = torch.cuda.CUDAGraph()
        ext.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g1, stream=ext):
            md.zero_()
            st_id = B.out_prod_id_back_status(ma.data_ptr(), moe.a_type, mg.data_ptr(), mi.data_ptr(),
                                              md.data_ptr(), moe.ne, moe.nb, raw)
        assert B.STATUS[st_id] == "E_CAPTURE"
        del g1
        torch.cuda.synchronize()
