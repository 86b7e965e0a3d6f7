"""out_prod_noalloc, the entry point that allocates nothing: split-K partials
in the library's static device scratch instead of a workspace of the pool.
Its result must equal out_prod's bit for bit (same plan, same summation
order), on consecutive calls of different sizes, under graph capture on a
stream that has no workspace, without the pool or the device's free memory
changing; a plan whose partials exceed the scratch is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from outer_product_gemm_amd import binding as B
from outer_product_gemm_amd import synth
from tests import gpu_util as G

SCRATCH_BYTES = 32 << 20


class Dev:
    """A workload's inputs on cuda:0 with an out_prod reference result."""

    def __init__(self, name):
        self.inst = i = synth.workload(name)
        self.a = G.to_dev(np.ascontiguousarray(i.a).view(np.uint8).reshape(-1))
        self.b = G.to_dev(i.b)
        self.out = torch.full(i.dst_shape, float("nan"), dtype=torch.float32, device="cuda:0")
        self.plan = B.out_prod_plan(self.a.data_ptr(), i.a_type, self.b.data_ptr(), self.out.data_ptr(),
                                    i.ne, i.nb)

    def args(self):
        i = self.inst
        return (self.a.data_ptr(), i.a_type, self.b.data_ptr(), self.out.data_ptr(), i.ne, i.nb)

    def result(self):
        torch.cuda.synchronize()
        return self.out.cpu().numpy()


@pytest.mark.gpu
def test_noalloc_matches_out_prod_on_consecutive_calls():
    """Two splitting calls in a row, the second smaller (the 4B input
    gradient: 4 K ranges, 21 MB of partials; then the rank-8 activation
    gradient: 8 ranges, 128 KB), then a call without a split: each equals
    out_prod's result bit for bit and passes the parity gate."""
    assert torch.cuda.is_available()
    B.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    big, small, plain = Dev("lora4B_dxW"), Dev("lora4B_dh"), Dev("deltanet_bcast")
    assert big.plan["splits"] > 1 and small.plan["splits"] > 1 and plain.plan["splits"] == 1
    assert small.plan["workspace_bytes"] < big.plan["workspace_bytes"] <= SCRATCH_BYTES
    refs = []
    for d in (big, small, plain):
        B.out_prod(*d.args(), stream)
        refs.append(d.result())
    # warm call: the first use on this device looks up the scratch's address
    B.out_prod_noalloc(*small.args(), stream)
    torch.cuda.synchronize()
    n_ws = B.out_prod_workspace_count()
    free0 = torch.cuda.mem_get_info()[0]
    for rep in range(2):
        for d, ref in zip((big, small, plain), refs):
            d.out.fill_(float("nan"))
            torch.cuda.synchronize()
            G.log("noalloc", d.inst.name, "rep", rep, "splits", d.plan["splits"])
            B.out_prod_noalloc(*d.args(), stream)
            got = d.result()
            assert np.array_equal(got, ref), (d.inst.name, rep)
            if rep == 0:
                i = d.inst
                r, den = oracle.out_prod(i.a, i.a_type, i.b, i.ne, i.nb)
                res = oracle.check(got, r, den, 1e-5)
                assert res["ok"], (d.inst.name, res)
    assert B.out_prod_workspace_count() == n_ws
    # (the HIP runtime may map a few MiB of its own on first use of a path)
    assert torch.cuda.mem_get_info()[0] >= free0 - (8 << 20)


@pytest.mark.gpu
def test_noalloc_under_graph_capture():
    """Captured on a fresh stream that holds no workspace, a splitting
    out_prod_noalloc keeps its split (out_prod would fall back to the unsplit
    plan there): every replay equals out_prod's eager result bit for bit,
    with eager work on the captured buffers between replays."""
    B.load_library()
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    raw = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(raw)) == 0
    try:
        ext = torch.cuda.ExternalStream(raw.value)
        big, small = Dev("lora4B_dxW"), Dev("lora4B_dh")
        cur = torch.cuda.current_stream().cuda_stream
        refs = []
        for d in (big, small):
            B.out_prod(*d.args(), cur)
            refs.append(d.result())
        B.out_prod_noalloc(*small.args(), cur)   # first use on this device outside capture
        torch.cuda.synchronize()
        n_ws = B.out_prod_workspace_count()
        g = torch.cuda.CUDAGraph()
        ext.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=ext):
            B.out_prod_noalloc(*big.args(), raw.value)
            B.out_prod_noalloc(*small.args(), raw.value)
        torch.cuda.synchronize()
        assert B.out_prod_workspace_count() == n_ws
        scale = 1.0
        for rep in range(4):
            big.out.fill_(float("nan"))
            small.out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(big.result(), refs[0] * np.float32(scale)), rep
            assert np.array_equal(small.result(), refs[1] * np.float32(scale)), rep
            big.b.mul_(2.0)
            small.b.mul_(2.0)
            scale *= 2.0
        del g
        torch.cuda.synchronize()
    finally:
        torch.cuda.synchronize()
        B.out_prod_release_stream(raw.value)
        hip.hipStreamDestroy(raw)


def test_noalloc_refuses_partials_beyond_the_scratch():
    """A plan whose split partials exceed the 32 MiB scratch (a q4_K weight of
    7168 x 16384 against 768 columns: 3 K ranges of 22 MB) is refused with
    E_SCRATCH on the host, before any HIP call (fake, never dereferenced
    addresses)."""
    ne, nb = synth.make_ne_nb(synth.Q4_K, (7168, 16384, 1, 1), (768, 16384, 1, 1))
    a, b, d = 1 << 28, 1 << 36, 1 << 40
    p = B.out_prod_plan(a, synth.Q4_K, b, d, ne, nb)
    assert p["splits"] > 1 and p["workspace_bytes"] > SCRATCH_BYTES
    assert B.STATUS[B.out_prod_noalloc_status(a, synth.Q4_K, b, d, ne, nb)] == "E_SCRATCH"
    # and the ordinary checks come first
    bad = list(ne)
    bad[5] += 1
    assert B.STATUS[B.out_prod_noalloc_status(a, synth.Q4_K, b, d, bad, nb)] == "E_K"
