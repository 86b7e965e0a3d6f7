"""OUT_PROD throughput on one MI355X, with roofline and CPU-oracle baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
every launch of the workload (the default workload, the 27B q4_K weight x f32
gradient products in both orientations, is two launches: m5120 k17408 n1024
and m17408 k5120 n1024).  Inputs are resident in HBM before timing starts;
R copies of them rotate so that consecutive steps do not hit the 256 MB
Infinity Cache.  Timing: W untimed warmup steps; K eager steps (reported as
ms_per_step_eager, host submission included); then exactly K steps captured
in one HIP graph and replayed between two synchronizations, timed with HIP
events on the stream the kernels run on.

Prints ONE JSON line (progress goes to stderr).  ``value`` is GFLOP/s of the
whole step; ``roofline`` reports the dominant kernel's algorithmic rate per
launch against the MI355X peak (fp32 MFMA 157.3 TFLOP/s, HBM 8 TB/s);
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from outer_product_gemm_amd import synth  # noqa: E402

METRIC = "OUT_PROD GFLOP/s and GB/s vs roofline, LoRA-backward shapes, 1×MI355X"
PEAK_MFMA_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
RIDGE = PEAK_MFMA_F32_TFLOPS * 1e3 / PEAK_HBM_GBPS   # flop per byte

COMPOSITE = {
    "q4_K_27B_both": ["q4_K_5120x17408", "q4_K_17408x5120"],
    # all four of the pages' per-op q4_K training shapes (n = 1024)
    "q4_K_page_shapes": ["q4_K_1536x1536", "q4_K_5120x5120", "q4_K_5120x17408", "q4_K_17408x5120"],
}
# The five OUT_PRODs of one LoRA-adapted linear layer's backward (frozen q4_K
# weight, rank 8): input gradient through W and through A, the gradient of
# the rank-8 activation, and the two adapter gradients.
COMPOSITE.update({name: list(group) for name, group in synth.LORA_BACKWARD.items()})
# Every frozen-weight a type at the 27B up-projection shape, one launch each.
COMPOSITE["a_types_5120x17408"] = list(synth.TYPE_SWEEP)
# ... and at m17408 k5120 n1024 (the 272 x 128 tile with loader waves).
COMPOSITE["a_types_17408x5120"] = list(synth.TYPE_SWEEP_DOWN)
# MUL_MAT_ID_BACK through q4_K experts: the up and down projections' input
# gradients of one mixture-of-experts FFN (64 experts, 8 routed, 512 tokens).
COMPOSITE["moe_back_q4_K"] = list(synth.MOE_WORKLOADS)
# The rank-4/8/24 LoRA parameter gradients at the 4B's widths (b of 2560 and
# 9216 columns, K = 512 tokens): one launch each, HBM-bound.
COMPOSITE["lora_rank_r"] = ["lora_r4_2560", "lora_r8_2560", "lora_r24_2560",
                            "lora_r4_9216", "lora_r8_9216", "lora_r24_9216"]
DEFAULT_WORKLOAD = "q4_K_27B_both"

# The pages' per-op float-staging times for the same q4_K x f32 shapes
# (Apple M5, Metal; "metal: OUT_PROD multiplies in float staging", review
# answer on cost): midpoints of 88-94, 88-90, 2.8-2.9 and 26-27 ms.  Another
# machine: context for vs_baseline only.
PAGE_MS = {"q4_K_5120x17408": 91.0, "q4_K_17408x5120": 89.0, "q4_K_1536x1536": 2.85,
           "q4_K_5120x5120": 26.5}

# HBM traffic per launch from rocprofv3 PMC runs (FETCH_SIZE + WRITE_SIZE,
# scaled by the copy-kernel calibration), keyed by workload, valid only for
# the kernel sources whose hash is recorded with it.
MEASURED_TRAFFIC = {
    # profiles/tiled_q4K_27B_lora_backward.md: launch A 378.4 MB, launch B 353.2 MB
    "q4_K_27B_both": {"kernel_hash": "bd4f5f101ce88df0", "bytes_per_launch": 365.82e6,
                      "profile": "profiles/tiled_q4K_27B_lora_backward.md"},
    # profiles/tiled_q4K_page_shapes.md: the four tiled launches (the m1536 split's
    # reduce kernel separate): 29.4 + 252.9 x 2 (m5120 k5120 and m5120 k17408, one
    # kernel group) + 353.2 MB
    "q4_K_page_shapes": {"kernel_hash": "bd4f5f101ce88df0", "bytes_per_launch": 222.12e6,
                         "profile": "profiles/tiled_q4K_page_shapes.md"},
    # profiles/tiled_q8_0_5120.md
    "q8_0_5120": {"kernel_hash": "bd4f5f101ce88df0", "bytes_per_launch": 167.2e6,
                  "profile": "profiles/tiled_q8_0_5120.md"},
    # profiles/lora_linear_backward_4B_27B.md: the tiled launches (split dx_W main kernel
    # 68.4 MB and dx_A 5.6 MB); the split's reduce kernel is reported there separately
    "lora_4B_linear_backward": {"kernel_hash": "bd4f5f101ce88df0", "bytes_per_launch": 37.03e6,
                                "profile": "profiles/lora_linear_backward_4B_27B.md"},
    # profiles/column_lora_rank_and_deltanet.md
    "lora_rank_r": {"kernel_hash": "d685f4d4c7ceb36c", "bytes_per_launch": 12.642e6,
                    "profile": "profiles/column_lora_rank_and_deltanet.md"},
    "lora_r8_9216": {"kernel_hash": "d685f4d4c7ceb36c", "bytes_per_launch": 19.41e6,
                     "profile": "profiles/column_lora_rank_and_deltanet.md"},
    "lora_r8_single": {"kernel_hash": "d685f4d4c7ceb36c", "bytes_per_launch": 5.56e6,
                       "profile": "profiles/column_lora_rank_and_deltanet.md"},
    "deltanet_bcast": {"kernel_hash": "d685f4d4c7ceb36c", "bytes_per_launch": 7.45e6,
                       "profile": "profiles/column_lora_rank_and_deltanet.md"},
    # profiles/id_back_moe_q4_K.md: the grouped tiled launches (routing kernel separate)
    "moe_back_q4_K": {"kernel_hash": "7766b790bf07e422", "bytes_per_launch": 155.01e6,
                      "profile": "profiles/id_back_moe_q4_K.md"},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources each kernel family's code and launch plan come from (the host
# file api.cpp chooses the plan; the family files hold the kernels).
FAMILY_SOURCES = {
    "tiled": ["api.cpp", "outprod_internal.h", "kernel_common.h", "block_formats.h", "tiled_impl.h",
              "kernel_tiled.hip", "tiled_f32.hip", "tiled_half.hip", "tiled_q8.hip", "tiled_q45.hip",
              "tiled_k4.hip", "tiled_k.hip", "kernel_reduce.hip"],
    "skinny": ["api.cpp", "outprod_internal.h", "kernel_common.h", "kernel_skinny.hip",
               "kernel_reduce.hip"],
}
FAMILY_SOURCES["tiled_id"] = FAMILY_SOURCES["tiled"] + ["kernel_id_back.hip"]


def kernel_source_hash(files=None):
    """Hash of the code (not the comments) of the given csrc files (default:
    every kernel and host source)."""
    from outer_product_gemm_amd.build import source_hash
    return source_hash(files)


def is_moe(inst):
    return isinstance(inst, synth.MoeInstance)


def make_instance(name):
    return synth.moe_workload(name) if name in synth.MOE_WORKLOADS else synth.workload(name)


def algorithmic(inst):
    """flops and bytes of one launch: 2*ne00*ne10*K*slices; unique a at its
    stored size (a broadcast a slice counts once) + b + one dst write.
    MUL_MAT_ID_BACK: 2*ne00*K per routed slot; the experts that some slot uses
    at their stored size + g + ids + dst."""
    ne = inst.ne
    if is_moe(inst):
        slots = ne[5] * ne[6]
        used = len(np.unique(inst.ids))
        a_bytes = synth.row_bytes(inst.a_type, ne[0]) * ne[1] * used
        return 2 * ne[0] * ne[1] * slots, a_bytes + 4 * slots * (ne[1] + 1 + ne[0])
    slices = ne[10] * ne[11]
    flops = 2 * ne[0] * ne[4] * ne[1] * slices
    a_bytes = synth.row_bytes(inst.a_type, ne[0]) * ne[1] * ne[2] * ne[3]
    b_bytes = 4 * ne[4] * ne[1] * ne[6] * ne[7]
    d_bytes = 4 * ne[0] * ne[4] * slices
    return flops, a_bytes + b_bytes + d_bytes


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(list(synth.WORKLOADS) + list(synth.MOE_WORKLOADS) + list(COMPOSITE)))
    ap.add_argument("--rotate", type=int, default=0, help="input copies (0 = enough for 600 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU-oracle time for the baseline sample (0 = skip)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="instead of the benchmark: run a plain device copy of MB megabytes "
                         "5 times (the reference for scaling HBM byte counters)")
    ap.add_argument("--peaks", action="store_true",
                    help="instead of the benchmark: measure the device's sustained fp32 MFMA, "
                         "HBM read and HBM copy rates and print them as JSON")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the short in-run measurement of the sustained peaks")
    ap.add_argument("--read-floor", action="store_true",
                    help="instead of the benchmark: time cold single-launch reads of the "
                         "workload's b (each f32 launch of it) in every strip decomposition of "
                         "the read-floor probe, and print the fastest per launch as JSON")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.peaks:
        print(json.dumps(measure_peaks(verbose=True)), flush=True)
        return
    if args.read_floor:
        read_floor(args.workload, args.steps)
        return

    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from outer_product_gemm_amd import binding as B

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    B.load_library()
    dev = torch.device("cuda:0")
    names = COMPOSITE.get(args.workload, [args.workload])
    log("workload", args.workload, names)

    insts = [make_instance(n) for n in names]
    work = [algorithmic(i) for i in insts]
    flops_step = sum(w[0] for w in work)
    bytes_step = sum(w[1] for w in work)
    launch_bytes = [i.a.nbytes + (i.g.nbytes + i.ids.nbytes if is_moe(i) else i.b.nbytes) +
                    4 * int(np.prod(i.dst_shape)) for i in insts]
    set_bytes = sum(launch_bytes)
    # Each launch rotates over enough copies of its own inputs (>= 600 MB of
    # them) that every timed launch, also in the per-launch pass below, reads
    # them from HBM rather than the 256 MB Infinity Cache.
    if args.rotate:
        copies_n = [args.rotate] * len(insts)
    else:
        copies_n = [max(1, min(256, int(np.ceil(600e6 / nb_)))) for nb_ in launch_bytes]
    R = max(copies_n)

    copies = []
    for j, inst in enumerate(insts):
        cj = []
        for r in range(copies_n[j]):
            a_d = torch.from_numpy(np.ascontiguousarray(inst.a).view(np.uint8).reshape(-1)).to(dev)
            if is_moe(inst):
                g_d = torch.from_numpy(inst.g).to(dev)
                i_d = torch.from_numpy(inst.ids).to(dev)
                d_d = torch.empty(inst.dst_shape, dtype=torch.float32, device=dev)
                plan = B.out_prod_id_back_plan(a_d.data_ptr(), inst.a_type, g_d.data_ptr(),
                                               i_d.data_ptr(), d_d.data_ptr(), inst.ne, inst.nb)
                plan["kernel_name"] = "tiled_id"
                cj.append((a_d, (g_d, i_d), d_d, plan))
                continue
            b_d = torch.from_numpy(inst.b).to(dev)
            d_d = torch.empty(inst.dst_shape, dtype=torch.float32, device=dev)
            plan = B.out_prod_plan(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), d_d.data_ptr(),
                                   inst.ne, inst.nb)
            cj.append((a_d, b_d, d_d, plan))
        copies.append(cj)
    # sets[r][j]: launch j's inputs for step r
    sets = [[copies[j][r % copies_n[j]] for j in range(len(insts))] for r in range(R)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    log("rotating copies per launch", copies_n, "set MB %.1f" % (set_bytes / 1e6),
        "plans", [(p[3]["kernel_name"], p[3]["tile_m"], p[3]["tile_n"], p[3]["grid"]) for p in sets[0]])

    def launch(r, j, stream_ptr):
        inst = insts[j]
        a_d, b_d, d_d, _ = sets[r][j]
        if is_moe(inst):
            B.out_prod_id_back(a_d.data_ptr(), inst.a_type, b_d[0].data_ptr(), b_d[1].data_ptr(),
                               d_d.data_ptr(), inst.ne, inst.nb, stream_ptr)
            return
        B.out_prod(a_d.data_ptr(), inst.a_type, b_d.data_ptr(), d_d.data_ptr(), inst.ne, inst.nb,
                   stream_ptr)

    for s in range(args.warmup):
        for j in range(len(insts)):
            launch(s % R, j, sptr)
    torch.cuda.synchronize()

    # Eager launches, one event pair per step (host submission included).
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for s in range(K):
        ev[s][0].record(stream)
        for j in range(len(insts)):
            launch(s % R, j, sptr)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms_eager = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))

    # Timed region: exactly K steps captured in one HIP graph (the library's
    # launches are recorded on the capturing stream), so small kernels are
    # not limited by host submission.  One untimed replay uploads the graph.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    # one uncaptured step on the capture stream first: a launch that splits K
    # allocates that stream's workspace on its first call
    for j in range(len(insts)):
        launch(0, j, cap.cuda_stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        cptr = torch.cuda.current_stream(dev).cuda_stream
        for s in range(K):
            for j in range(len(insts)):
                launch(s % R, j, cptr)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / K
    log("timed %d steps (graph): %.4f ms/step; eager %.4f ms/step (host wall %.3f s)"
        % (K, ms_step, ms_eager, wall))

    # Per-launch durations: each launch of the step alone, K times in a graph
    # of its own (rotating inputs as above), timed with HIP events.
    launch_us = []
    for j in range(len(insts)):
        g = torch.cuda.CUDAGraph()
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap):
            cptr = torch.cuda.current_stream(dev).cuda_stream
            for s in range(K):
                launch(s % R, j, cptr)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        launch_us.append(t0.elapsed_time(t1) / K * 1e3)
        del g
    log("per-launch us:", ["%s %.2f" % (i.name, u) for i, u in zip(insts, launch_us)])

    # Dominant kernel: the kernel family with the largest share of the step.
    # When every launch runs that family, its average launch duration is the
    # timed region's time per launch; otherwise it is the per-launch pass's.
    kname = [p[3]["kernel_name"] for p in sets[0]]
    share = {k: sum(u for u, n in zip(launch_us, kname) if n == k) for k in set(kname)}
    dom = max(share, key=share.get)
    sel = [j for j in range(len(insts)) if kname[j] == dom]
    flops_launch = np.array([work[j][0] for j in sel], dtype=np.float64)
    bytes_launch = np.array([work[j][1] for j in sel], dtype=np.float64)
    ai = flops_launch.sum() / bytes_launch.sum()
    bound = "mfma" if ai >= RIDGE else "hbm"
    kernels = [dom]
    # algorithmic work per launch / the kernel's average launch duration
    if len(sel) == len(insts):
        mean_s = ms_step / len(insts) * 1e-3
    else:
        mean_s = float(np.mean([launch_us[j] for j in sel])) * 1e-6
    if bound == "mfma":
        achieved = float(flops_launch.mean()) / mean_s / 1e12
        peak, unit = PEAK_MFMA_F32_TFLOPS, "TFLOP/s"
    else:
        achieved = float(bytes_launch.mean()) / mean_s / 1e9
        peak, unit = PEAK_HBM_GBPS, "GB/s"
    src_hash = kernel_source_hash()
    fam_hash = kernel_source_hash(FAMILY_SOURCES.get(dom))
    traffic = None
    mt = MEASURED_TRAFFIC.get(args.workload)
    if mt and mt.get("kernel_hash") == fam_hash:
        traffic = int(mt["bytes_per_launch"])
        traffic_source = ("rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of this workload (L2-to-"
                          "memory bytes, Infinity Cache hits included), scaled by a 256 MB copy's "
                          "counts, recorded for the %s kernel sources with hash %s (%s)"
                          % (dom, fam_hash, mt["profile"]))
    elif mt:
        traffic_source = ("none: the %s kernel sources (hash %s) changed since the counters were "
                          "taken (hash %s)" % (dom, fam_hash, mt["kernel_hash"]))
    else:
        traffic_source = "none: no counter run recorded for this workload"
    measured = None if args.no_peaks else measure_peaks()
    roofline = {
        "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
        "frac": round(achieved / peak, 4), "traffic": traffic, "traffic_source": traffic_source,
        "kernel": dom,
        "launches_of_kernel": [insts[j].name for j in sel],
        "avg_launch_us": round(mean_s * 1e6, 3),
        "algorithmic_flops_per_launch": [int(x) for x in flops_launch],
        "algorithmic_bytes_per_launch": [int(x) for x in bytes_launch],
    }
    if measured is not None:
        mp = measured["mfma_f32_tflops"] if bound == "mfma" else measured["hbm_read_gbps"]
        roofline["measured_peak"] = round(mp, 3)
        roofline["frac_of_measured_peak"] = round(achieved / mp, 4)
        roofline["measured_peak_note"] = (
            "this device's sustained rate in the same run: %s" %
            ("a loop of independent v_mfma_f32_32x32x2_f32" if bound == "mfma" else
             "a 4 GiB streaming read"))

    # NaN/Inf in the outputs of the last step (every launch's whole dst)
    nonfinite = 0
    for j in range(len(insts)):
        d = sets[(K - 1) % R][j][2]
        nonfinite += int(d.numel() - torch.isfinite(d).sum().item())

    value = flops_step / (ms_step * 1e-3) / 1e9
    gbps = bytes_step / (ms_step * 1e-3) / 1e9
    vs = None
    if all(n in PAGE_MS for n in names):
        page_gflops = flops_step / (sum(PAGE_MS[n] for n in names) * 1e-3) / 1e9
        vs = round(value / page_gflops, 2)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(insts, sets, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": vs,
        "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": args.workload,
            "launches": [{"name": i.name, "a_type": synth.TYPE_NAMES[i.a_type],
                          "ne00": i.ne[0], "K": i.ne[1],
                          **({"op": "mul_mat_id_back", "n_expert": i.ne[2], "n_used": i.ne[5],
                              "n_tokens": i.ne[6]} if is_moe(i) else
                             {"ne10": i.ne[4], "slices": i.ne[10] * i.ne[11],
                              "b_layout": "k_contiguous" if i.b_kt else "row"}),
                          "kernel": p[3]["kernel_name"], "variant": p[3]["variant"],
                          "swapped": bool(p[3].get("swapped", 0)), "us": round(u, 3)}
                         for i, p, u in zip(insts, sets[0], launch_us)],
            "rotating_input_copies": copies_n,
        },
        "gbps": round(gbps, 1),
        "ms_per_step_eager": round(ms_eager, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_source_hash": src_hash,
        "kernel_family_hash": fam_hash,
        "git_rev": git_rev(),
        "library_build": library_build(src_hash),
        "seeds": {i.name: int(i.seed) for i in insts},
        "nonfinite_outputs": nonfinite,
        "measured_peaks": measured,
    }
    if vs is not None:
        out["vs_baseline_note"] = ("ratio to the pages' float-staging per-op times for the same "
                                   "shapes on an Apple M5 (Metal): another machine, context only")
    print(json.dumps(out), flush=True)


def git_rev():
    from outer_product_gemm_amd.build import git_rev as rev
    return rev()


def library_build(src_hash):
    """What the loaded liboutprod.so was built from (its build stamp): the
    sources' code hash then, whether it equals the sources' hash now, and the
    commit checked out at build time (the only revision a tree copied without
    git metadata carries)."""
    from outer_product_gemm_amd.build import read_stamp
    stamp = read_stamp()
    if stamp is None:
        log("warning: liboutprod.so has no build stamp")
        return None
    ok = stamp.get("source_hash") == src_hash
    if not ok:
        log("warning: liboutprod.so was built from sources with hash %s, the sources now hash to %s"
            % (stamp.get("source_hash"), src_hash))
    return {"source_hash": stamp.get("source_hash"), "matches_sources": ok,
            "git_rev_at_build": stamp.get("git_rev")}


def load_calib():
    import ctypes
    import torch  # noqa: F401  (the HIP runtime torch loads must come first)
    path = os.path.join(ROOT, "outer_product_gemm_amd", "libcalib.so")
    if not os.path.exists(path):
        raise SystemExit("libcalib.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.calib_mfma_f32.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    lib.calib_read.argtypes = [vp, i64, vp, ctypes.c_int, vp]
    lib.calib_copy.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.calib_strip_read.argtypes = [vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, vp, vp]
    return lib


def _time_graph(fn, reps):
    """Mean ms of one call of fn(stream_ptr), from `reps` calls captured in one
    graph and replayed once (after one untimed replay)."""
    import torch
    dev = torch.device("cuda:0")
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    fn(cap.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        sp = torch.cuda.current_stream(dev).cuda_stream
        for _ in range(reps):
            fn(sp)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st = torch.cuda.current_stream(dev)
    t0.record(st)
    g.replay()
    t1.record(st)
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) / reps


def measure_peaks(verbose=False):
    """Sustained rates of this device, each from a graph of back-to-back
    launches timed with HIP events: fp32 MFMA (2048 workgroups x 4 waves, each
    wave 4 independent v_mfma_f32_32x32x2_f32 chains of 2048 steps: 275 GFLOP
    per launch), a 4 GiB streaming read, and a 1 GiB device copy (counted as
    read + write bytes)."""
    import torch
    lib = load_calib()
    dev = torch.device("cuda:0")
    grid, iters = 2048, 2048
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    flops = grid * 4 * iters * 4 * 4096
    ms = _time_graph(lambda sp: lib.calib_mfma_f32(out.data_ptr(), grid, iters, sp), 10)
    mfma = flops / (ms * 1e-3) / 1e12
    n_read = (4 << 30) // 16
    src = torch.ones(n_read * 4, dtype=torch.float32, device=dev)
    rgrid = 256 * 16
    rout = torch.empty(rgrid * 256, dtype=torch.float32, device=dev)
    ms_r = _time_graph(lambda sp: lib.calib_read(src.data_ptr(), n_read, rout.data_ptr(), rgrid, sp), 10)
    read = n_read * 16 / (ms_r * 1e-3) / 1e9
    n_copy = (1 << 30) // 16
    dst = torch.empty(n_copy * 4, dtype=torch.float32, device=dev)
    ms_c = _time_graph(lambda sp: lib.calib_copy(src.data_ptr(), dst.data_ptr(), n_copy, rgrid, sp), 10)
    copy = 2 * n_copy * 16 / (ms_c * 1e-3) / 1e9
    del src, dst, out, rout
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    res = {"mfma_f32_tflops": mfma, "mfma_ms": ms, "hbm_read_gbps": read, "read_ms": ms_r,
           "hbm_copy_gbps": copy, "copy_ms": ms_c,
           "datasheet": {"mfma_f32_tflops": PEAK_MFMA_F32_TFLOPS, "hbm_gbps": PEAK_HBM_GBPS}}
    if verbose:
        log("peaks: mfma %.1f TFLOP/s (%.3f ms), read %.0f GB/s (%.3f ms), copy %.0f GB/s (%.3f ms)"
            % (mfma, ms, read, ms_r, copy, ms_c))
    return res


def read_floor(workload, reps):
    """The read floor of each f32 launch of a workload: for its b ([K][N] fp32
    rows), every strip decomposition of the probe (strips of 16-256 columns,
    K ranges, 256 or 512 threads, 4-16 loads in flight per thread), each timed
    as `reps` launches in a graph over rotating cold copies (enough for 600 MB,
    past the 256 MB Infinity Cache).  Prints one JSON line: per launch, the
    fastest configuration and the times of all."""
    import torch
    lib = load_calib()
    dev = torch.device("cuda:0")
    names = COMPOSITE.get(workload, [workload])
    report, seen = [], set()
    for name in names:
        inst = make_instance(name)
        if is_moe(inst) or inst.b_kt:
            continue
        ne = inst.ne
        N, K = ne[4] * ne[6] * ne[7], ne[1]
        if N > 65536 or (K, N) in seen:
            continue
        seen.add((K, N))
        plane = 4 * N * K
        R = max(2, int(np.ceil(600e6 / plane)))
        bufs = [torch.randn(K, N, dtype=torch.float32, device=dev) for _ in range(R)]
        results = []
        for cols in (16, 32, 64, 128, 256):
            if N % cols:
                continue
            for threads in (256, 512):
                if cols // 4 > threads:
                    continue
                for krows in sorted({K, max(1, K // 2), max(1, K // 4), max(1, K // 8)}, reverse=True):
                    wgs = (N // cols) * ((K + krows - 1) // krows)
                    if wgs > 8192:
                        continue
                    for U in (4, 8, 16):
                        out = torch.empty(wgs * threads, dtype=torch.float32, device=dev)
                        it = [0]

                        def fn(sp, cols=cols, threads=threads, krows=krows, U=U, out=out):
                            b = bufs[it[0] % R]
                            it[0] += 1
                            rc = lib.calib_strip_read(b.data_ptr(), 4 * N, K, N, cols, krows, threads, U,
                                                      out.data_ptr(), sp)
                            if rc != 0:
                                raise RuntimeError("calib_strip_read %d" % rc)
                        ms = _time_graph(fn, reps)
                        results.append({"cols": cols, "threads": threads, "krows": krows, "U": U,
                                        "workgroups": wgs, "us": round(ms * 1e3, 3)})
        results.sort(key=lambda r: r["us"])
        best = results[0]
        log("%s: b %d x %d (%.2f MB): fastest %s; %.0f GB/s" % (
            name, K, N, plane / 1e6, best, plane / (best["us"] * 1e-6) / 1e9))
        report.append({"name": name, "K": K, "N": N, "b_bytes": plane, "best": best,
                       "best_gbps": round(plane / (best["us"] * 1e-6) / 1e9, 1),
                       "all": results})
        del bufs
        torch.cuda.empty_cache()
    print(json.dumps({"read_floor": report}), flush=True)


def copy_calibration(mb):
    """A plain device-to-device copy of known size, 5 times: under rocprofv3
    --pmc its FETCH_SIZE / WRITE_SIZE per dispatch against the known bytes give
    the factor that scales those counters to HBM bytes."""
    import torch
    n = int(mb * 1e6) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                      "copies": 5}), flush=True)


def cpu_baseline(insts, sets, target_s):
    """Time the CPU oracle, as it stands, on a bounded sample of the same
    workload: all ne00 outputs of some dst columns (routed slots for
    MUL_MAT_ID_BACK) of every launch.  The sample grows until one pass takes
    at least 80% of target_s or covers every launch's whole output; a pass
    shorter than that is repeated on the same sample until the total does.
    The same columns of the GPU result are checked against it (max error
    ratio reported)."""
    import oracle
    import torch  # noqa: F401

    threads = oracle.num_threads()
    rng = np.random.default_rng(123)

    def pick(n):
        """The sample: per launch, up to n columns (slots); and whether that
        is every launch's whole output."""
        picks, whole = [], True
        for inst in insts:
            ne = inst.ne
            if is_moe(inst):
                n_slots = ne[5] * ne[6]
                cnt = min(n, n_slots)
                whole = whole and cnt == n_slots
                picks.append(np.sort(rng.choice(n_slots, cnt, replace=False)))
            else:
                tot = ne[4] * ne[10] * ne[11]
                cnt = min(n, tot)
                whole = whole and cnt == tot
                flat = rng.choice(tot, cnt, replace=False)
                picks.append(np.array([[c % ne[4], (c // ne[4]) % ne[10], c // (ne[4] * ne[10])]
                                       for c in flat]))
        return picks, whole

    def run(picks):
        t_all, f_all, results = 0.0, 0, []
        for j, (inst, sel) in enumerate(zip(insts, picks)):
            ne = inst.ne
            t = time.perf_counter()
            if is_moe(inst):
                ref, den = oracle.mul_mat_id_back(inst.a, inst.a_type, inst.g, inst.ids, ne,
                                                  inst.nb, slots=sel)
            else:
                ref, den = oracle.out_prod(inst.a, inst.a_type, inst.b, ne, inst.nb, cols=sel)
            t_all += time.perf_counter() - t
            f_all += 2 * ne[0] * ne[1] * len(sel)
            results.append((j, sel, ref, den))
        return t_all, f_all, results

    n = max(1, threads // 2)
    while True:
        picks, whole = pick(n)
        t_all, f_all, results = run(picks)
        log("cpu oracle sample: %d columns/launch, %.2f s" % (n, t_all))
        if t_all >= 0.8 * target_s or whole or n >= (1 << 20):
            break
        n = int(n * min(8.0, max(1.5, target_s / max(t_all, 1e-3))))
    total_t, total_flops, reps = t_all, f_all, 1
    while total_t < 0.8 * target_s and reps < 100000:
        t_rep, f_rep, _ = run(picks)
        total_t += t_rep
        total_flops += f_rep
        reps += 1
    if reps > 1:
        log("cpu oracle sample repeated %d times, %.2f s" % (reps, total_t))
    sample_desc, worst = [], 0.0
    for j, cols, ref, den in results:
        d = sets[0][j][2].cpu().numpy()
        if is_moe(insts[j]):
            nu = insts[j].ne[5]
            g = np.stack([d[s // nu, s % nu] for s in cols])
            sample_desc.append("%s: %d routed slots x %d" % (insts[j].name, len(cols), insts[j].ne[0]))
        else:
            g = np.stack([d[i3, i2, i1] for i1, i2, i3 in cols])
            sample_desc.append("%s: %d dst columns x %d" % (insts[j].name, len(cols), insts[j].ne[0]))
        worst = max(worst, oracle.check(g, ref, den)["max_ratio"])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        cpu_model = platform.processor()
    return {
        "value": round(total_flops / total_t / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": "; ".join(sample_desc) + " (double accumulation%s, %.1f s)" % (
            ", %d passes" % reps if reps > 1 else "", total_t),
        "cpu_model": cpu_model,
        "sample_parity_max_ratio": worst,
    }


if __name__ == "__main__":
    main()
