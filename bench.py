"""Benchmark: GPU weight decode of the 276-matrix DiT-shaped stack on one MI355X.

One step = decode every matrix of the stack (6 281 625 600 BF16 parameters,
target 4.0 bpp) from its resident compressed blob into its own BF16 buffer,
block by block: one launch per transformer block (9 matrices: q, k, v, o, w1,
w3, w2, mod1, mod2), 31 launches per step.  Inputs are seeded synthetic
matrices drawn on the GPU and compressed by the library's host encoder before
timing; blobs and output buffers are resident in HBM when the timed region
starts.

Printed as one JSON line: value = BF16 output GB/s of the whole step; also the
HBM roofline of the decode kernel (algorithmic bytes = compressed bytes read +
BF16 bytes written, per launch, over the HIP-event launch time), the oracle
decoder timed on the host, the per-layer (one launch per matrix) variant and the
fused compressed-linear prefill overhead (14336 x 4096 weight, 4096 tokens).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
VALU_LANE_OPS_PER_S = 256 * 64 * 2.4e9   # 256 CUs, 4 SIMDs x 16 lanes each, 2.4 GHz


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--target-bpp", type=float, default=4.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-linear", action="store_true")
    p.add_argument("--no-layer-mode", action="store_true")
    p.add_argument("--no-lossless", action="store_true")
    p.add_argument("--no-gpu-encode", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="skip the 8192^2 container and chains-per-tile sweep")
    p.add_argument("--matrices", type=int, default=276, help="first N matrices of the stack (profiling runs)")
    p.add_argument("--streams", type=int, default=3, help="HIP streams the block launches rotate over")
    p.add_argument("--chains-per-tile", type=int, default=0,
                   help="chains per tile of the stack's blobs (0: the encoder's choice, 8 for these sizes)")
    p.add_argument("--gemm-only", action="store_true",
                   help="only run the BF16 and FP8 GEMMs at 4096 x 14336 x 4096 and hipBLASLt (counter runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (to scale HBM byte counters)")
    return p.parse_args()


def copy_calibration(reps=5):
    """A plain copy kernel of known size: FETCH_SIZE / WRITE_SIZE of this run give the
    counter scale (bytes moved per counted KiB) for the decode kernel's traffic."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": reps}))


def gemm_only(reps=5):
    """Counter runs: our BF16 GEMM, our FP8 GEMM and hipBLASLt (torch.matmul) on the prefill
    shape, T x N x K = 4096 x 14336 x 4096, `reps` calls each, one after the other."""
    import torch
    import synth
    from decode_tile_rans_amd import _lib as L
    T, N, K = 4096, 14336, 4096
    x = torch.from_numpy(synth.activations(T, K, 50)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(synth.rowscaled(N, K, 5)).view(torch.bfloat16).cuda()
    wq, aw = synth.fp8_codes(N, K, 5)
    xq, axr = synth.fp8_codes(T, K, 50)
    wqt, xqt, awt = torch.from_numpy(wq).cuda(), torch.from_numpy(xq).cuda(), torch.from_numpy(aw).cuda()
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    sp = int(torch.cuda.current_stream().cuda_stream)
    for _ in range(reps):
        L.ep_gemm_bf16_nt(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), T, N, K, sp)
    for _ in range(reps):
        L.ep_gemm_fp8_nt(xqt.data_ptr(), wqt.data_ptr(), float(axr.max()), awt.data_ptr(), y.data_ptr(), T, N, K, sp)
    for _ in range(reps):
        torch.matmul(x, w.t())
    torch.cuda.synchronize()
    print(json.dumps({"gemm_only": [T, N, K], "reps": reps}))


def practical_ceilings(reps=10):
    """Achievable HBM rates on this GPU as context for the decode's byte rate: a plain
    1 GiB device copy (read + write) and a 1 GiB fill (write only), torch's own kernels."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    st = torch.cuda.current_stream()

    def rate(fn, bytes_moved):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return round(bytes_moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    out = {"copy_GBps": rate(lambda: b.copy_(a), 2 * n), "write_only_GBps": rate(lambda: b.fill_(2), n)}
    del a, b
    torch.cuda.empty_cache()
    return out


def container_sweep(reps=10):
    """One 8192 x 8192 matrix (log-normal row scales, seed 4; FP8 / INT8 per-row absmax
    codes of it): decode time per container and target bitrate, warm (back to back) and
    cold (a 512 MB write between launches evicts the 256 MB last-level cache); then the
    chains-per-tile sweep at BF16 4.0 bpp (state bits per tile against parallelism)."""
    import torch
    import synth
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    n = 8192
    st = torch.cuda.current_stream()
    sp = int(st.cuda_stream)
    junk = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def times(c, out_t):
        dst = torch.empty((n, n), dtype=out_t, device="cuda")
        for _ in range(3):
            L.ep_decompress(c.handle, dst.data_ptr(), sp)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            L.ep_decompress(c.handle, dst.data_ptr(), sp)
        b.record(st)
        torch.cuda.synchronize()
        warm = a.elapsed_time(b) / reps
        cold = 0.0
        for _ in range(reps):
            junk.fill_(1)
            a.record(st)
            L.ep_decompress(c.handle, dst.data_ptr(), sp)
            b.record(st)
            torch.cuda.synchronize()
            cold += a.elapsed_time(b) / reps
        return warm, cold

    def entry(c, out_t, esz, **kw):
        warm, cold = times(c, out_t)
        alg = c.nbytes + esz * n * n
        return dict(kw, actual_bpp=round(c.actual_bpp, 4), ms_warm=round(warm, 4), ms_cold=round(cold, 4),
                    out_GBps_warm=round(esz * n * n / (warm * 1e-3) / 1e9, 1),
                    hbm_frac_warm=round(alg / (warm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    hbm_frac_cold=round(alg / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))

    os.environ["EP_NUM_THREADS"] = str(min(16, os.cpu_count() or 1))
    out = {"containers": [], "chains_per_tile": []}
    bf = synth.rowscaled(n, n, 4)
    for kind, t in (("bf16", 2.3), ("bf16", 3.0), ("bf16", 5.0), ("bf16", 8.0), ("fp8", 5.0), ("int8", 4.0)):
        if kind == "bf16":
            c, out_t, esz = ep.compress(bf, t, dtype=torch.bfloat16), torch.bfloat16, 2
        elif kind == "fp8":
            c, out_t, esz = ep.compress(synth.fp8_codes(n, n, 4)[0], t, dtype=torch.float8_e4m3fn), torch.float8_e4m3fn, 1
        else:
            c, out_t, esz = ep.compress(synth.int8_codes(n, n, 4)[0], t, dtype=torch.int8), torch.int8, 1
        c.upload()
        out["containers"].append(entry(c, out_t, esz, container=kind, target_bpp=t))
        del c
    for S in (1, 2, 4, 8):
        c = ep.compress(bf, 4.0, dtype=torch.bfloat16, chains_per_tile=S)
        c.upload()
        out["chains_per_tile"].append(entry(c, torch.bfloat16, 2, S=S))
        del c
    os.environ.pop("EP_NUM_THREADS", None)
    del junk
    torch.cuda.empty_cache()
    return out


def build_stack(n, target_bpp, chains_per_tile=0):
    """Draw the stack on the GPU and compress it there (the GPU encoder's batch entry,
    whose blobs equal the host encoder's byte for byte), upload the blobs."""
    import torch
    import synth
    import decode_tile_rans_amd as ep
    shapes = synth.dit_stack_shapes()[:n]
    t0 = time.time()
    comps = []
    for i0 in range(0, n, 32):
        ws = [synth.dit_stack_torch(i) for i in range(i0, min(n, i0 + 32))]
        comps += ep.compress_many(ws, target_bpp, chains_per_tile=chains_per_tile)
        del ws
    for c in comps:
        c.upload()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"compressed {n} matrices in {time.time() - t0:.1f}s on the GPU")
    blocks = {}
    for i, (_, _, _, b) in enumerate(shapes):
        blocks.setdefault(b, []).append(i)
    return comps, [blocks[b] for b in sorted(blocks)]


_SIDE_STREAMS = []


def time_stack(comps, blocks, outs, steps, warmup, per_layer=False, n_streams=1):
    """Time `steps` passes over the stack.  Consecutive launches rotate over n_streams
    streams (default priority) so one launch's tail overlaps the next one's start; every
    pass ends with all streams joined."""
    import torch
    from decode_tile_rans_amd import _lib as L
    main = torch.cuda.current_stream()
    # side streams are created once per process and reused: each new HIP stream is bound
    # to one of the runtime's few hardware queues in turn, and a side stream that shares
    # the main stream's queue would serialise with it
    while len(_SIDE_STREAMS) < n_streams - 1:
        _SIDE_STREAMS.append(torch.cuda.Stream())
    streams = [main] + _SIDE_STREAMS[:n_streams - 1]
    handles = [c.handle for c in comps]
    ptrs = [o.data_ptr() for o in outs]
    units = [[i] for i in range(len(comps))] if per_layer else blocks

    def launch(k, u):
        sp = int(streams[k % n_streams].cuda_stream)
        if len(u) == 1:
            L.ep_decompress(handles[u[0]], ptrs[u[0]], sp)
        else:
            L.ep_decompress_batch([handles[i] for i in u], [ptrs[i] for i in u], sp)

    def fork():
        ev = torch.cuda.Event()
        ev.record(main)
        for s in streams[1:]:
            s.wait_event(ev)

    def join():
        for s in streams[1:]:
            ev = torch.cuda.Event()
            ev.record(s)
            main.wait_event(ev)

    for _ in range(warmup):
        fork()
        for k, u in enumerate(units):
            launch(k, u)
        join()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in units]
    t0 = time.perf_counter()
    for s in range(steps):
        fork()
        for k, u in enumerate(units):
            st = streams[k % n_streams]
            if s == steps - 1:
                ev[k][0].record(st)
            launch(k, u)
            if s == steps - 1:
                ev[k][1].record(st)
        join()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    return wall / steps * 1e3, launch_ms, units


_COUNTERS_APPLY = [True]   # false when the stack's blobs differ from the counted ones


def decode_counters():
    """The committed rocprofv3 counter summary of the decode kernel (HBM bytes and VALU
    instructions per parameter), or None when the kernel source changed since then (or
    the stack is encoded with another chain count than the counted one)."""
    import hashlib
    if not _COUNTERS_APPLY[0]:
        return None
    try:
        info = json.load(open(os.path.join(ROOT, "profiles", "decode_traffic.json")))
        src = open(os.path.join(ROOT, "decode_tile_rans_amd", "csrc", "decode.hip"), "rb").read()
    except OSError:
        return None
    if hashlib.sha1(src).hexdigest() != info.get("decode_source_sha1"):
        return None
    return info


def traffic_per_launch(coords_per_launch):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE, or None (see decode_counters)."""
    info = decode_counters()
    if info is None:
        return None
    return (info["fetch_bytes_per_param"] + info["write_bytes_per_param"]) * coords_per_launch


def valu_issue(params_per_s, key="valu_lane_ops_per_param"):
    """The decode against the chip's VALU issue rate (256 CUs x 64 lanes x 2.4 GHz lane
    operations per second) at the measured SQ_INSTS_VALU x 64 lane operations per
    parameter of the kernel variant `key` names (the roofline launch's two chains per
    lane, or the timed step's one); None without a current counter summary."""
    info = decode_counters()
    if info is None or key not in info:
        return None
    ops = info[key]
    ceiling = VALU_LANE_OPS_PER_S / ops
    return {"lane_ops_per_param": ops, "peak_lane_ops_per_s": VALU_LANE_OPS_PER_S,
            "ceiling_params_per_s": round(ceiling), "achieved_params_per_s": round(params_per_s),
            "frac": round(params_per_s / ceiling, 4)}


def _oracle_decode_worker(args):
    """One host process of the oracle baseline: decode the blob repeatedly for about
    `seconds`; returns (coordinates decoded, seconds)."""
    blob, n_coords, seconds = args
    import oracle
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.decode(blob)
        n += n_coords
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_bpp, seconds=10.0):
    """The oracle decoder (NumPy) on one 3840 x 3840 stack matrix: one process, then one
    process per host core (at most 16, the host share of one GPU) each decoding the
    blob for the same time; the all-cores rate is the reported value."""
    import multiprocessing as mp
    import numpy as np
    import oracle
    import synth
    from oracle import numerics as nx
    w = synth.dit_stack_torch(0).cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    blob = oracle.compress(w, nx.DT_BF16, target_bpp)
    n1, dt1 = _oracle_decode_worker((blob, w.size, seconds))
    nproc = os.cpu_count() or 1
    workers = max(1, min(16, nproc))
    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map(_oracle_decode_worker, [(blob, w.size, 0.0)] * workers)     # start-up and imports
        t0 = time.perf_counter()
        res = pool.map(_oracle_decode_worker, [(blob, w.size, seconds)] * workers)
        wall = time.perf_counter() - t0
    n_all = sum(n for n, _ in res)
    return {"value": round(2.0 * n_all / wall / 1e9, 4), "unit": "GB/s (BF16 out)", "cores": workers, "kind": "oracle",
            "sample": f"oracle.decode of one 3840x3840 stack matrix (14.7M params) in {workers} processes for "
                      f"{wall:.1f}s ({n_all // w.size} decodes), NumPy",
            "coords_per_s": round(n_all / wall, 1), "nproc": nproc, "cpu_model": _cpu_model(),
            "single_process": {"value": round(2.0 * n1 / dt1 / 1e9, 4), "coords_per_s": round(n1 / dt1, 1),
                               "seconds": round(dt1, 1), "cores": 1}}


def fused_linear(target_bpp, reps=10):
    """CompressedLinear prefill: W 14336x4096 (row-scaled, seed 5), X 4096x4096 N(0,1) (seed 50)."""
    import numpy as np
    import torch
    import synth
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    R, C, T = 14336, 4096, 4096
    wbits = synth.rowscaled(R, C, 5)
    os.environ["EP_NUM_THREADS"] = str(min(16, os.cpu_count() or 1))
    c = ep.compress(wbits, target_bpp, dtype=torch.bfloat16)
    os.environ.pop("EP_NUM_THREADS", None)
    c.upload()
    x = torch.from_numpy(synth.activations(T, C, 50)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(wbits).view(torch.bfloat16).cuda()
    y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    need = L.ep_linear_workspace_bytes(c.handle)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()
    sp = int(st.cuda_stream)
    wd = ws.data_ptr() + ((256 - ws.data_ptr() % 256) % 256)

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    fns = {
        "fused": lambda: L.ep_compressed_linear_forward(c.handle, x.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(),
                                                        need, sp),
        "dec": lambda: L.ep_decompress(c.handle, wd, sp),
        "gemm": lambda: L.ep_gemm_bf16_nt(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), T, R, C, sp),
        "torch": lambda: torch.matmul(x, w.t()),
    }
    # the GPU's clocks settle over the first few hundred milliseconds of MFMA load: run the
    # GEMM until then, and take each variant's best of three rounds measured in turn
    for _ in range(40):
        fns["gemm"]()
    torch.cuda.synchronize()
    best = {k: min(timeit(f) for _ in range(3)) for k, f in fns.items()}
    for _ in range(2):
        for k, f in fns.items():
            best[k] = min(best[k], timeit(f))
    t_fused, t_dec, t_gemm, t_torch = best["fused"], best["dec"], best["gemm"], best["torch"]
    flops = 2.0 * T * R * C
    # a sequence of layers (4 distinct weights, each twice): the next layer's decode on a
    # second stream while this layer's GEMM runs, against the same GEMMs on plain weights
    seq = linear_sequence(c, wbits, target_bpp, timeit)
    small = small_batch(c, w, x, ws, need, wd, sp, timeit)
    prefill = prefill_fused(c, w, x, wd, sp, timeit)
    sweep = token_sweep(c, w, ws, need, sp, timeit)
    s16 = chains_per_tile_8_vs_16(c, w, x, target_bpp, sp, timeit)
    return {
        "workload": "CompressedLinear prefill 14336x4096 weight @%.1f bpp, 4096 tokens" % target_bpp,
        "actual_bpp": round(c.actual_bpp, 4),
        "ms_decode_plus_gemm": round(t_fused, 4), "ms_decode": round(t_dec, 4), "ms_gemm_plain_bf16": round(t_gemm, 4),
        "ms_torch_matmul_hipblaslt": round(t_torch, 4),
        "overhead_pct_vs_our_gemm": round(100.0 * (t_fused / t_gemm - 1.0), 2),
        "overhead_pct_vs_hipblaslt": round(100.0 * (t_fused / t_torch - 1.0), 2),
        "gemm_mfma_util": round(flops / (t_gemm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "gemm_tflops": round(flops / (t_gemm * 1e-3) / 1e12, 1),
        "sequence_overlapped": seq,
        "small_batch": small,
        "prefill_fused": prefill,
        "token_sweep": sweep,
        "chains_per_tile_8_vs_16": s16,
    }


def chains_per_tile_8_vs_16(c8, w, x, target_bpp, sp, timeit):
    """The same weight encoded with 16 chains per tile instead of 8: half the symbols per
    chain (a lone launch is bound by that depth) for a larger blob.  Lone decode, the
    one-token product and decode + GEMM at the activations' token count, the two blobs
    timed in alternating rounds (best of three each)."""
    import torch
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    R, C = w.shape
    T = x.shape[0]
    c16 = ep.compress(w, target_bpp, chains_per_tile=16, stream=torch.cuda.current_stream())
    c16.upload()
    need = max(L.ep_linear_workspace_bytes(c.handle) for c in (c8, c16))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dec = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((1, R), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    fns = {}
    for S, c in ((8, c8), (16, c16)):
        h = c.handle
        fns[(S, "ms_decode")] = lambda h=h: L.ep_decompress(h, dec.data_ptr(), sp)
        fns[(S, "ms_fused_1_token")] = lambda h=h: L.ep_compressed_linear_forward(
            h, x.data_ptr(), 1, None, y1.data_ptr(), ws.data_ptr(), need, sp)
        fns[(S, "ms_decode_plus_gemm")] = lambda h=h: L.ep_compressed_linear_forward(
            h, x.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(), need, sp)
    fns[("plain", "ms_gemm_plain_bf16")] = lambda: L.ep_gemm_bf16_nt(x.data_ptr(), w.data_ptr(), None, y.data_ptr(),
                                                                     T, R, C, sp)
    best = {k: float("inf") for k in fns}
    for _ in range(3):
        for k, f in fns.items():
            best[k] = min(best[k], timeit(f))
    torch.cuda.synchronize()
    if c16.device_errors():
        raise SystemExit("decode of the 16-chain blob reported failed chains")
    out = {"tokens": T, "ms_gemm_plain_bf16": round(best[("plain", "ms_gemm_plain_bf16")], 4)}
    for S, c in ((8, c8), (16, c16)):
        out[f"chains_{S}"] = {"actual_bpp": round(c.actual_bpp, 4),
                              **{k: round(v, 4) for (s, k), v in best.items() if s == S}}
    return out


def token_sweep(c, w, ws, need, sp, timeit):
    """The compressed linear (decode, then our GEMM) against our plain GEMM on the same
    weight for 512 .. 16384 tokens (X N(0,1), seed 51): the decode's share shrinks as the
    product grows."""
    import torch
    import synth
    from decode_tile_rans_amd import _lib as L
    R, C = c.shape
    out = []
    for T in (512, 1024, 2048, 4096, 8192, 16384):
        x = torch.from_numpy(synth.activations(T, C, 51)).view(torch.bfloat16).cuda()
        y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        fused = lambda: L.ep_compressed_linear_forward(c.handle, x.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(),
                                                       need, sp)
        plain = lambda: L.ep_gemm_bf16_nt(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), T, R, C, sp)
        t_f, t_p = timeit(fused), timeit(plain)
        for _ in range(2):
            t_f, t_p = min(t_f, timeit(fused)), min(t_p, timeit(plain))
        out.append({"tokens": T, "ms_decode_plus_gemm": round(t_f, 4), "ms_gemm": round(t_p, 4),
                    "overhead_pct": round(100.0 * (t_f / t_p - 1.0), 2)})
        del x, y
    return out


def prefill_fused(c, w, x, wd, sp, timeit):
    """The same layer on 16..256 tokens: the fused prefill product (each K slab of W decoded
    into an LDS operand tile of the MFMA product; weights never written; what
    ep_compressed_linear_forward takes at these sizes) against decode to memory then our
    GEMM, our GEMM alone and hipBLASLt on the plain BF16 weight."""
    import torch
    from decode_tile_rans_amd import _lib as L
    R, C = c.shape
    out = []

    def best(fn):
        return min(timeit(fn) for _ in range(3))

    for T in (16, 32, 64, 128, 192, 256):
        xs = x[:T].contiguous()
        y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        t_mma = best(lambda: L.ep_compressed_linear_prefill(c.handle, xs.data_ptr(), T, None, y.data_ptr(), sp))
        t_two = best(lambda: (L.ep_decompress(c.handle, wd, sp),
                                L.ep_gemm_bf16_nt(xs.data_ptr(), wd, None, y.data_ptr(), T, R, C, sp)))
        t_gemm = best(lambda: L.ep_gemm_bf16_nt(xs.data_ptr(), w.data_ptr(), None, y.data_ptr(), T, R, C, sp))
        t_plain = best(lambda: torch.matmul(xs, w.t()))
        out.append({"tokens": T, "ms_fused_prefill": round(t_mma, 4), "ms_decode_then_gemm": round(t_two, 4),
                    "ms_our_gemm_plain_bf16": round(t_gemm, 4), "ms_hipblaslt_plain_bf16": round(t_plain, 4),
                    "fused_speedup_vs_decode_then_gemm": round(t_two / t_mma, 3),
                    "fused_tflops": round(2.0 * T * R * C / (t_mma * 1e-3) / 1e12, 1),
                    "fused_blob_gbs": round(c.nbytes / (t_mma * 1e-3) / 1e9, 1)})
    # a weight of 8192 columns (two tiles a row): 8192 x 8192 @4.0 (seed 6)
    import synth
    import decode_tile_rans_amd as ep
    os.environ["EP_NUM_THREADS"] = str(min(16, os.cpu_count() or 1))
    c2 = ep.compress(synth.rowscaled(8192, 8192, 6), 4.0, dtype=torch.bfloat16)
    os.environ.pop("EP_NUM_THREADS", None)
    c2.upload()
    R2, C2 = c2.shape
    x2 = torch.from_numpy(synth.activations(256, C2, 53)).view(torch.bfloat16).cuda()
    w2 = torch.empty((R2, C2), dtype=torch.bfloat16, device="cuda")
    L.ep_decompress(c2.handle, w2.data_ptr(), sp)
    wd2 = torch.empty((R2, C2), dtype=torch.bfloat16, device="cuda")
    out2 = []
    for T in (16, 64, 128, 256):
        xs = x2[:T].contiguous()
        y = torch.empty((T, R2), dtype=torch.bfloat16, device="cuda")
        t_mma = best(lambda: L.ep_compressed_linear_prefill(c2.handle, xs.data_ptr(), T, None, y.data_ptr(), sp))
        t_two = best(lambda: (L.ep_decompress(c2.handle, wd2.data_ptr(), sp),
                                L.ep_gemm_bf16_nt(xs.data_ptr(), wd2.data_ptr(), None, y.data_ptr(), T, R2, C2, sp)))
        t_gemm = best(lambda: L.ep_gemm_bf16_nt(xs.data_ptr(), w2.data_ptr(), None, y.data_ptr(), T, R2, C2, sp))
        out2.append({"tokens": T, "ms_fused_prefill": round(t_mma, 4), "ms_decode_then_gemm": round(t_two, 4),
                     "ms_our_gemm_plain_bf16": round(t_gemm, 4),
                     "fused_speedup_vs_decode_then_gemm": round(t_two / t_mma, 3)})
    return {"layer_14336x4096": out, "layer_8192x8192": out2}


def small_batch(c, w, x, ws, need, wd, sp, timeit):
    """The same layer on 1..8 tokens (decode-time inference): the fused decode-and-product
    kernel against decode then our GEMM and against hipBLASLt on the plain BF16 weight.
    Rate = blob bytes / fused time (the weights are read once, compressed)."""
    import torch
    from decode_tile_rans_amd import _lib as L
    R, C = c.shape
    out = []

    def best(fn):
        return min(timeit(fn) for _ in range(3))

    for T in (1, 2, 4, 5, 8):
        xs = x[:T].contiguous()
        y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        nmv = L.ep_matvec_workspace_bytes(c.handle, T)
        t_mv = best(lambda: L.ep_compressed_matvec(c.handle, xs.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(),
                                                     nmv, sp))
        t_pf = best(lambda: L.ep_compressed_linear_prefill(c.handle, xs.data_ptr(), T, None, y.data_ptr(), sp))
        t_two = best(lambda: (L.ep_decompress(c.handle, wd, sp),
                                L.ep_gemm_bf16_nt(xs.data_ptr(), wd, None, y.data_ptr(), T, R, C, sp)))
        t_plain = best(lambda: torch.matmul(xs, w.t()))
        out.append({"tokens": T, "ms_fused": round(t_mv, 4), "ms_fused_prefill_kernel": round(t_pf, 4),
                    "ms_decode_then_gemm": round(t_two, 4), "ms_hipblaslt_plain_bf16": round(t_plain, 4),
                    "fused_speedup_vs_decode_then_gemm": round(t_two / t_mv, 3),
                    "fused_blob_gbs": round(c.nbytes / (t_mv * 1e-3) / 1e9, 1),
                    "plain_weight_gbs": round(2.0 * R * C / (t_plain * 1e-3) / 1e9, 1)})
    return {"layer_14336x4096": out, "qkv_3840": qkv_batch(timeit, sp)}


def qkv_batch(timeit, sp):
    """Query, key and value projections of one 3840-wide layer (three 3840 x 3840 weights
    @4.0 bpp, seeds 900..902) on one token: three fused calls against one batched call."""
    import torch
    import synth
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    os.environ["EP_NUM_THREADS"] = str(min(16, os.cpu_count() or 1))
    cs = [ep.compress(synth.rowscaled(3840, 3840, 900 + i), 4.0, dtype=torch.bfloat16) for i in range(3)]
    os.environ.pop("EP_NUM_THREADS", None)
    for c in cs:
        c.upload()
    hs = [c.handle for c in cs]
    out = {}
    for T in (1, 8):
        x = torch.randn(T, 3840, dtype=torch.bfloat16, device="cuda")
        ys = [torch.empty((T, 3840), dtype=torch.bfloat16, device="cuda") for _ in cs]
        n1 = L.ep_matvec_workspace_bytes(hs[0], T)
        nb = L.ep_matvec_batch_workspace_bytes(hs, T)
        ws = torch.empty(max(n1, nb), dtype=torch.uint8, device="cuda")
        t_sep = min(timeit(lambda: [L.ep_compressed_matvec(h, x.data_ptr(), T, None, y.data_ptr(), ws.data_ptr(), n1, sp)
                                for h, y in zip(hs, ys)]) for _ in range(3))
        t_bat = min(timeit(lambda: L.ep_compressed_matvec_batch(hs, x.data_ptr(), T, None, [y.data_ptr() for y in ys],
                                                            ws.data_ptr(), nb, sp)) for _ in range(3))
        out[f"tokens_{T}"] = {"ms_three_calls": round(t_sep, 4), "ms_batched": round(t_bat, 4),
                              "speedup": round(t_sep / t_bat, 3)}
    return out


def linear_sequence(c0, wbits0, target_bpp, timeit, n_layers=8):
    """n_layers compressed linears of the 14336x4096 shape (weights of seeds 5..8 in
    turn) at 4096 and at 256 tokens (X N(0,1), seed 52): serial (decode then GEMM per
    layer, one stream), the sequence entry (which puts the decode of layer i+1 on a side
    stream beside the GEMM of layer i when that GEMM leaves CUs idle: at 256 tokens its
    56 tiles use 56 of the 256 CUs; at 4096 tokens it fills them and the entry runs in
    order) and plain BF16 GEMMs."""
    import torch
    import synth
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    R, C = wbits0.shape
    comps, wts = [c0], [torch.from_numpy(wbits0).view(torch.bfloat16).cuda()]
    os.environ["EP_NUM_THREADS"] = str(min(16, os.cpu_count() or 1))
    for seed in (6, 7, 8):
        wb = synth.rowscaled(R, C, seed)
        c = ep.compress(wb, target_bpp, dtype=torch.bfloat16)
        c.upload()
        comps.append(c)
        wts.append(torch.from_numpy(wb).view(torch.bfloat16).cuda())
    os.environ.pop("EP_NUM_THREADS", None)
    layers = [i % len(comps) for i in range(n_layers)]
    hs = [comps[i].handle for i in layers]
    out = {}
    for T in (4096, 256):
        x = torch.from_numpy(synth.activations(T, C, 52)).view(torch.bfloat16).cuda()
        out[f"tokens_{T}"] = _sequence_times(L, hs, wts, layers, x, T, R, C, n_layers, timeit)
    del wts
    return out


def _sequence_times(L, hs, wts, layers, x, T, R, C, n_layers, timeit):
    import torch
    ys = [torch.empty((T, R), dtype=torch.bfloat16, device="cuda") for _ in layers]
    st = torch.cuda.current_stream()
    sp = int(st.cuda_stream)
    if not _SIDE_STREAMS:
        _SIDE_STREAMS.append(torch.cuda.Stream())
    side = _SIDE_STREAMS[0]      # (the first side stream: not on the main stream's queue)
    need = L.ep_linear_seq_workspace_bytes(hs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    n1 = L.ep_linear_workspace_bytes(hs[0])
    ws1 = torch.empty(n1, dtype=torch.uint8, device="cuda")

    def plain():
        for i, y in zip(layers, ys):
            L.ep_gemm_bf16_nt(x.data_ptr(), wts[i].data_ptr(), None, y.data_ptr(), T, R, C, sp)

    def serial():
        for h, y in zip(hs, ys):
            L.ep_compressed_linear_forward(h, x.data_ptr(), T, None, y.data_ptr(), ws1.data_ptr(), n1, sp)

    def overlapped():
        L.ep_compressed_linear_seq_forward(hs, [x.data_ptr()] * n_layers, T, None, [y.data_ptr() for y in ys],
                                           ws.data_ptr(), need, sp, int(side.cuda_stream))

    # best of three rounds measured in turn (clocks drift over a run)
    t_plain, t_serial, t_over = timeit(plain), timeit(serial), timeit(overlapped)
    for _ in range(2):
        t_plain, t_serial, t_over = min(t_plain, timeit(plain)), min(t_serial, timeit(serial)), \
            min(t_over, timeit(overlapped))
    del ys, ws, ws1
    return {"layers": n_layers, "tokens": T, "ms_plain_bf16_gemms": round(t_plain, 4), "ms_serial": round(t_serial, 4),
            "ms_sequence_entry": round(t_over, 4), "side_stream_used": (T + 255) // 256 * ((R + 255) // 256) < 256,
            "overhead_pct_serial": round(100.0 * (t_serial / t_plain - 1.0), 2),
            "overhead_pct_sequence_entry": round(100.0 * (t_over / t_plain - 1.0), 2)}


def lossless_block(reps=10):
    """TileANS (lossless) on the first 9-matrix DiT block: raw BF16 bytes compressed on the
    host, decoded in one batched launch per pass."""
    import torch
    import synth
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    t0 = time.time()
    comps = [ep.compress_lossless(synth.dit_stack_torch(i).cpu()) for i in range(9)]
    t_enc = time.time() - t0
    for c in comps:
        c.upload()
    outs = [torch.empty(c.shape, dtype=c.dtype, device="cuda") for c in comps]
    sp = int(torch.cuda.current_stream().cuda_stream)
    n_el = sum(o.numel() for o in outs)
    cbytes = sum(c.nbytes for c in comps)

    def run():
        L.ep_decompress_batch([c.handle for c in comps], [o.data_ptr() for o in outs], sp)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    if sum(c.device_errors() for c in comps):
        raise SystemExit("lossless decode reported failed chains")
    ok = all(torch.equal(o.cpu().view(torch.int16), synth.dit_stack_torch(i).cpu().view(torch.int16))
             for i, o in enumerate(outs))
    if not ok:
        raise SystemExit("lossless decode differs from its input")
    alg = cbytes + 2 * n_el
    return {"workload": "TileANS lossless, first 9-matrix DiT block (BF16, 206M params), one batched launch",
            "bits_per_param": round(8.0 * cbytes / n_el, 4), "ratio": round(16.0 * n_el / (8.0 * cbytes), 4),
            "ms_decode": round(ms, 4), "bf16_out_GBps": round(2 * n_el / (ms * 1e-3) / 1e9, 1),
            "algorithmic_GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "host_encode_s": round(t_enc, 2), "bit_exact": ok}


def fp8_linear(reps=10):
    """FP8@5 ([README]/[NEWS]: FP8 W8A8 weight codes compressed at 5 bpp, FP8 GEMM): decode
    the 14336x4096 code tensor to FP8, then the FP8 MFMA GEMM with 4096 FP8 activations."""
    import torch
    import synth
    import decode_tile_rans_amd as ep
    from decode_tile_rans_amd import _lib as L
    R, C, T = 14336, 4096, 4096
    wq, aw = synth.fp8_codes(R, C, 5)
    xq, ax_rows = synth.fp8_codes(T, C, 50)
    c = ep.compress(wq, 5.0, dtype=torch.float8_e4m3fn)
    c.upload()
    wd = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    xt = torch.from_numpy(xq).cuda()
    awt = torch.from_numpy(aw).cuda()
    y = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    a_x = float(ax_rows.max())
    st = torch.cuda.current_stream()
    sp = int(st.cuda_stream)

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def gemm():
        L.ep_gemm_fp8_nt(xt.data_ptr(), wd.data_ptr(), a_x, awt.data_ptr(), y.data_ptr(), T, R, C, sp)

    for _ in range(40):   # settle the clocks under MFMA load
        gemm()
    torch.cuda.synchronize()
    fns = [lambda: L.ep_decompress(c.handle, wd.data_ptr(), sp), gemm,
           lambda: (L.ep_decompress(c.handle, wd.data_ptr(), sp), gemm())]
    t_dec, t_gemm, t_both = [min(timeit(f) for _ in range(3)) for f in fns]
    flops = 2.0 * T * R * C
    return {"workload": "FP8@5: 14336x4096 E4M3FN weight codes @5.0 bpp, FP8 GEMM with 4096 FP8 tokens",
            "actual_bpp": round(c.actual_bpp, 4), "ms_decode": round(t_dec, 4), "ms_fp8_gemm": round(t_gemm, 4),
            "ms_decode_plus_gemm": round(t_both, 4), "fp8_gemm_tflops": round(flops / (t_gemm * 1e-3) / 1e12, 1),
            "fp8_mfma_util": round(flops / (t_gemm * 1e-3) / 1e12 / 5000.0, 4),
            "overhead_pct": round(100.0 * (t_both / t_gemm - 1.0), 2)}


def gpu_encode_stack(n, target_bpp):
    """The GPU encoder over the stack: every matrix already in HBM (BF16), compressed by
    the batch entry (and, for comparison, one call per matrix on one stream); wall time
    of the whole pass against the host encoder's rate on a few matrices (all host cores)."""
    import torch
    import synth
    from decode_tile_rans_amd import _lib as L
    ws = [synth.dit_stack_torch(i) for i in range(n)]
    torch.cuda.synchronize()
    sp = int(torch.cuda.current_stream().cuda_stream)
    h = L.ep_compress_device(ws[0].data_ptr(), L.EP_BF16, ws[0].shape[0], ws[0].shape[1], target_bpp, 0, sp)
    L.ep_blob_free(h)
    t0 = time.time()
    nbytes = 0
    for w in ws:
        h = L.ep_compress_device(w.data_ptr(), L.EP_BF16, w.shape[0], w.shape[1], target_bpp, 0, sp)
        nbytes += L.ep_serialized_size(h)
        L.ep_blob_free(h)
    dt = time.time() - t0
    # the same matrices through the batch entry (four host threads, a stream each)
    t0 = time.time()
    hs_b = L.ep_compress_device_batch([w.data_ptr() for w in ws], [tuple(w.shape) for w in ws], L.EP_BF16,
                                      target_bpp, 0, sp)
    dt_batch = time.time() - t0
    nbytes_b = sum(L.ep_serialized_size(h) for h in hs_b)
    for h in hs_b:
        L.ep_blob_free(h)
    params = sum(w.numel() for w in ws)
    # host encoder on the first 9 matrices (one transformer block)
    hs = [w.cpu() for w in ws[:9]]
    t1 = time.time()
    for w in hs:
        h = L.ep_compress(w.data_ptr(), L.EP_BF16, w.shape[0], w.shape[1], target_bpp, 0)
        L.ep_blob_free(h)
    dh = time.time() - t1
    hp = sum(w.numel() for w in hs)
    return {"workload": f"GPU encoder, {n} stack matrices (BF16, resident in HBM), target {target_bpp} bpp",
            "seconds": round(dt_batch, 3), "params_per_s": round(params / dt_batch, 1),
            "actual_bpp": round(8.0 * nbytes / params, 4), "entry": "ep_compress_device_batch (4 host threads)",
            "seconds_one_call_per_matrix": round(dt, 3), "batch_bytes_equal": nbytes_b == nbytes,
            "host_encoder_params_per_s": round(hp / dh, 1), "host_threads": os.cpu_count()}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gemm_only:
        gemm_only()
        return
    comps, blocks = build_stack(a.matrices, a.target_bpp, a.chains_per_tile)
    _COUNTERS_APPLY[0] = comps[0].chains_per_tile == 8
    outs = [torch.empty(c.shape, dtype=torch.bfloat16, device="cuda") for c in comps]
    n_params = sum(c.shape[0] * c.shape[1] for c in comps)
    blob_bytes = sum(c.nbytes for c in comps)
    out_bytes = 2 * n_params

    ms, _, units = time_stack(comps, blocks, outs, a.steps, a.warmup, n_streams=a.streams)
    # per-launch kernel time for the roofline: one stream, launches back to back, each
    # launch alone on the GPU (so its blocks are spread evenly over the CUs, one
    # workgroup per CU: EP_DECODE_SPREAD=1); the same launches with the timed step's
    # shape (one block per wave, made for overlapping streams) reported beside it
    _, launch_ms_std, _ = time_stack(comps, blocks, outs, 2, 1, n_streams=1)
    os.environ["EP_DECODE_SPREAD"] = "1"
    _, launch_ms, _ = time_stack(comps, blocks, outs, 2, 1, n_streams=1)
    os.environ.pop("EP_DECODE_SPREAD", None)
    errs = sum(c.device_errors() for c in comps)
    if errs:
        raise SystemExit(f"decode reported {errs} failed chains")
    kern_ms = sum(launch_ms)
    alg_bytes = blob_bytes + out_bytes
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": "weight decode GB/s (BF16 out) & % HBM roofline; fused-linear overhead %",
        "value": round(out_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; trained weights unavailable)",
        "config": {"workload": f"{len(comps)}-matrix DiT-shaped BF16 stack (30 blocks x q,k,v,o 3840^2, w1,w3 "
                               f"10240x3840, w2 3840x10240, mod1,mod2 3840^2 + 6 x 3840^2), target "
                               f"{a.target_bpp} bpp, decoded block by block (one launch per 9-matrix block)",
                   "params": n_params, "compressed_bytes": blob_bytes,
                   "actual_bpp": round(8.0 * blob_bytes / n_params, 4),
                   "resident_bpp": round(8.0 * sum(c.device_bytes for c in comps) / n_params, 4),
                   "launches_per_step": len(units),
                   "streams": a.streams, "chains_per_tile": comps[0].chains_per_tile},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (lambda t: round(t) if t else None)(traffic_per_launch(n_params / len(units))),
                     "kernel": "decode_kernel (BF16 out)", "avg_launch_ms": round(kern_ms / len(units), 5),
                     "launch_shape": "one stream, blocks spread evenly over the CUs (EP_DECODE_SPREAD=1): the "
                                     "9-matrix launches at two chains per lane, every block resident at once",
                     "frac_one_block_per_wave": round(alg_bytes / (sum(launch_ms_std) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "avg_launch_ms_one_block_per_wave": round(sum(launch_ms_std) / len(units), 5),
                     "algorithmic_bytes_per_launch": round(alg_bytes / len(units)),
                     "step_effective_GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
                     "step_effective_frac": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "valu_issue_per_launch": valu_issue(n_params / (kern_ms * 1e-3)),
                     "valu_issue_step": valu_issue(n_params / (ms * 1e-3), "valu_lane_ops_per_param_step"),
                     "practical_ceilings": practical_ceilings()},
    }
    if not a.no_layer_mode:
        ms_l, lms, units_l = time_stack(comps, blocks, outs, max(2, a.steps // 2), 1, per_layer=True,
                                        n_streams=max(a.streams, 4))
        result["per_layer_mode"] = {"ms_per_step": round(ms_l, 4),
                                    "bf16_out_GBps": round(out_bytes / (ms_l * 1e-3) / 1e9, 2),
                                    # the step's algorithmic bytes over its wall time (the launches
                                    # overlap across streams, so their durations do not add up)
                                    "hbm_frac": round(alg_bytes / (ms_l * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                    "launches_per_step": len(units_l), "streams": max(a.streams, 4)}
    del outs
    torch.cuda.empty_cache()
    if not a.no_linear:
        result["fused_linear"] = fused_linear(a.target_bpp)
        result["fp8_linear"] = fp8_linear()
    if not a.no_lossless:
        result["lossless"] = lossless_block()
    if not a.no_gpu_encode:
        result["gpu_encode"] = gpu_encode_stack(a.matrices, a.target_bpp)
    if not a.no_sweep:
        result["sweep_8192"] = container_sweep()
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(a.target_bpp)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
