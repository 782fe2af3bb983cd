"""Benchmark of the Kimi K3 LatentMoE routed-expert layer on one MI355X.

A step is one pass of the whole layer (router, latent projection, dispatch, MXFP4
experts, combine + RMSNorm, up-projection) over one batch of synthetic input already
resident in HBM. The headline workload is the K3-shape decode layer: T = 1 token per
step, hidden 7168, latent 3584, inter 3072, 896 MXFP4 experts (15.7 GB resident),
top-16. Each step reads a different token from a pool of 64, so the routed experts
change from step to step, and the steps rotate over copies of the dense weights (4 by
default, 128 MB each), so those are not served from the 256 MB MALL either. Beside it:
the K3-shape prefill (T = 4096), the skewed prefill (T = 8192, 90 hot experts taking 80%
of the pairs), the layer at 8, 64 and 256 tokens, the shared experts, the two
approximate variants, and the CPU oracle on the host's cores.

Prints one JSON line (rank 0). Per-kernel times come from the same kind of steps run
through k3moe_layer_profiled, which binds a pair of HIP events to each kernel launch's
own start and end on the stream it runs on; a step's time is the sum over its launches.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix cores


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing enabled)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


MAX_LAUNCHES = 32  # timed kernel launches per profiled layer call, more than one layer call makes


def launch_ms(events: HipEvents, names):
    """Kernel time in ms per step name of one profiled call: launch i ran between
    events[2i] and events[2i+1]."""
    out = {}
    for i, n in enumerate(names):
        out[n] = out.get(n, 0.0) + events.ms(events.ev[2 * i], events.ev[2 * i + 1])
    return out


def figures_from_profile(name: str, key: str, kernel: str):
    """A per-kernel figure recorded in a committed counter summary (profiles/<name>), or
    None when the kernel sources have changed since the counters were taken (their sha256
    is recorded with the figures)."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    vals, srcs, sha = {}, [], None
    for line in lines:
        parts = line.split()
        if len(parts) == 3 and parts[0] == key:
            vals[parts[1]] = float(parts[2])
        elif parts and parts[0] == "kernel_sources":
            srcs = parts[1:]
        elif len(parts) == 2 and parts[0] == "kernel_source_sha256":
            sha = parts[1]
    h = hashlib.sha256()
    for src in srcs:
        try:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        except OSError:
            return None
    if sha is None or h.hexdigest() != sha:
        return None
    return vals.get(kernel)


def traffic_from_profile(kernel: str):
    """HBM-side bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE)."""
    v = figures_from_profile("expert_gateup_decode_T1_traffic.txt", "traffic_bytes_per_launch", kernel)
    return int(v) if v is not None else None


def algorithmic(dims, T, n_distinct):
    """Bytes the layer must move and flops it must do for one step: every distinct routed
    expert's record once, the dense weights once, the token's input and output; flops count
    the router, both projections and the three expert products of each (token, expert)
    pair, at 2 per multiply-add."""
    import k3gen
    H, L, I, E, K = dims.hidden, dims.latent, dims.inter, dims.n_experts, dims.topk
    blob = k3gen.ExpertLayout(dims).blob_bytes
    gateup_unit = 2 * (I * L // 2 + I * L // 32)     # w1 + w3 of one expert
    down_unit = L * I // 2 + L * I // 32             # w2 of one expert
    dense_bytes = E * H * 4 + L * H * 2 + H * L * 2 + E * 4 + L * 4
    act_bytes = T * H * 2 + T * H * 4
    flops = T * (2 * E * H + 2 * L * H + K * 2 * 3 * I * L + 2 * H * L)
    return {
        "layer_bytes": n_distinct * blob + dense_bytes + act_bytes,
        "gateup_bytes": n_distinct * gateup_unit,
        "down_bytes": n_distinct * down_unit,
        "flops": flops,
        "expert_flops": T * K * 2 * 3 * I * L,
    }


def bench_shared(args, dims, stream, xs, pool, row, hip_record, n_shared=2):
    """The fused shared experts (k3moe_shared_glu_bf16, y += on the layer output) at the
    K3 shape: decode (T = 1, rotating over two copies of the 264 MB of weights, so they
    come from HBM) and prefill (T = 4096)."""
    import torch

    import k3gen
    from mxfp4_routed_expert_amd import device, k3moe
    sh = k3gen.gen_shared(dims, 1, n_shared)
    copies = [device.upload_shared(sh)]
    copies.append({k: v.clone() for k, v in copies[0].items()})
    del sh
    SI, H = n_shared * dims.inter, dims.hidden
    w_bytes = 3 * SI * H * 2
    T = 1
    y = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    ws = device.shared_workspace(dims, n_shared, T)

    def call(i, **kw):
        c = copies[i % 2]
        return (k3moe.k3moe_shared_profiled if kw else k3moe.k3moe_shared_glu_bf16)(
            dims, n_shared, T, xs.data_ptr() + (i % pool) * row, c["sh1"], c["sh3"], c["sh2"], y, ws,
            stream=stream, **kw)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    ev = HipEvents(2)
    hip_record(ev.ev[0], stream.cuda_stream)
    for i in range(args.steps):
        call(i)
    hip_record(ev.ev[1], stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(ev.ev[0], ev.ev[1]) / args.steps
    ev.close()
    pe = HipEvents(2 * MAX_LAUNCHES)
    sums = {}
    nprof = min(args.steps, 50)
    for i in range(nprof):
        names = call(i, events=pe.ev)
        torch.cuda.synchronize()
        for n, v in launch_ms(pe, names).items():
            sums[n] = sums.get(n, 0.0) + v
    pe.close()
    kern = {n: round(v / nprof * 1e3, 2) for n, v in sums.items()}
    gbs = (w_bytes + H * 2 + 2 * H * 4) / (ms * 1e-3) / 1e9
    gu_us = kern.get("shared_gate_up_situ")
    gu_gbs = (2 * SI * H * 2) / (gu_us * 1e-6) / 1e9 if gu_us else None
    out = {"n_shared": n_shared, "inter": SI, "decode_us_per_step": round(ms * 1e3, 2),
           "decode_GBs": round(gbs, 1), "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "gate_up_GBs": round(gu_gbs, 1) if gu_gbs else None, "decode_kernel_us": kern}
    log(f"shared experts decode T=1: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s; per-kernel us: "
        + ", ".join(f"{n} {v:.1f}" for n, v in kern.items()))
    if not args.no_prefill:
        Tp = 4096
        xp = torch.from_numpy(k3gen.gen_x(dims, 3, Tp).view(np.int16)).cuda()
        yp = torch.zeros((Tp, H), dtype=torch.float32, device="cuda")
        wsp = device.shared_workspace(dims, n_shared, Tp)
        c = copies[0]
        k3moe.k3moe_shared_glu_bf16(dims, n_shared, Tp, xp, c["sh1"], c["sh3"], c["sh2"], yp, wsp, stream=stream)
        torch.cuda.synchronize()
        evp = HipEvents(2)
        hip_record(evp.ev[0], stream.cuda_stream)
        for _ in range(args.prefill_steps):
            k3moe.k3moe_shared_glu_bf16(dims, n_shared, Tp, xp, c["sh1"], c["sh3"], c["sh2"], yp, wsp,
                                        stream=stream)
        hip_record(evp.ev[1], stream.cuda_stream)
        torch.cuda.synchronize()
        msp = evp.ms(evp.ev[0], evp.ev[1]) / args.prefill_steps
        evp.close()
        pep = HipEvents(2 * MAX_LAUNCHES)
        names = k3moe.k3moe_shared_profiled(dims, n_shared, Tp, xp, c["sh1"], c["sh3"], c["sh2"], yp, wsp, pep.ev,
                                            stream=stream)
        torch.cuda.synchronize()
        kp = {n: round(v * 1e3, 1) for n, v in launch_ms(pep, names).items()}
        pep.close()
        tf = Tp * 2 * 3 * SI * H / (msp * 1e-3) / 1e12
        out.update({"prefill_T": Tp, "prefill_ms_per_step": round(msp, 3), "prefill_TFLOPs": round(tf, 1),
                    "prefill_bf16_peak_frac": round(tf / BF16_PEAK_TFLOPS, 4), "prefill_kernel_us": kp})
        log(f"shared experts prefill T=4096: {msp:.2f} ms/step, {tf:.0f} TFLOP/s (2 bf16 pieces of act "
            f"counted once); per-kernel us: " + ", ".join(f"{n} {v:.0f}" for n, v in kp.items()))
        del xp, yp, wsp
    del copies
    torch.cuda.empty_cache()
    return out


def time_block(step, n, stream, hip_record):
    """ms per step over n steps between one pair of events on the stream."""
    import torch
    ev = HipEvents(2)
    torch.cuda.synchronize()
    hip_record(ev.ev[0], stream.cuda_stream)
    for i in range(n):
        step(i)
    hip_record(ev.ev[1], stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(ev.ev[0], ev.ev[1]) / n
    ev.close()
    return ms


def time_each(step, n, stream, hip_record):
    """ms of each of n steps, one event pair around each (steps back to back)."""
    import torch
    ev = HipEvents(2 * n)
    torch.cuda.synchronize()
    for i in range(n):
        hip_record(ev.ev[2 * i], stream.cuda_stream)
        step(i)
        hip_record(ev.ev[2 * i + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    out = [ev.ms(ev.ev[2 * i], ev.ev[2 * i + 1]) for i in range(n)]
    ev.close()
    return out


def profiled_kernels(call, n):
    """Mean per-step-name kernel time (us) over n profiled calls; call(events) runs one."""
    import torch
    pe = HipEvents(2 * MAX_LAUNCHES)
    sums = {}
    for i in range(n):
        names = call(i, pe.ev)
        torch.cuda.synchronize()
        for k, v in launch_ms(pe, names).items():
            sums[k] = sums.get(k, 0.0) + v
    pe.close()
    return {k: round(v / n * 1e3, 2) for k, v in sums.items()}


def routing_stats(dims, idx: np.ndarray, hot=None):
    """Load balance of one batch's routing: tokens per expert, and the grouped GEMM's
    column tiles and their split over the XCDs (the kernels' own tiling)."""
    from mxfp4_routed_expert_amd import k3moe
    E = dims.n_experts
    counts = np.bincount(idx[idx >= 0].ravel(), minlength=E)
    out = {"distinct_experts": int(np.count_nonzero(counts)), "tokens_per_expert_max": int(counts.max()),
           "tokens_per_expert_median": float(np.median(counts)),
           "tokens_per_expert_mean": round(float(counts.mean()), 2)}
    if hot is not None:
        cold = counts[~hot]
        out.update({"hot_share": round(float(counts[hot].sum() / counts.sum()), 4),
                    "hot_tokens_mean": round(float(counts[hot].mean()), 1),
                    "cold_with_1_to_5_tokens": round(float(np.mean((cold >= 1) & (cold <= 5))), 4),
                    "cold_with_0_tokens": round(float(np.mean(cold == 0)), 4)})
    tile, rows_gu, rows_dn, small = k3moe.gemm_tiling()
    # the experts of at most `small` pairs take the decode kernel, the others column tiles
    out["experts_to_decode_kernel"] = int(np.count_nonzero((counts > 0) & (counts <= small)))
    out["pairs_to_decode_kernel"] = int(counts[(counts > 0) & (counts <= small)].sum())
    ncol = np.where(counts > small, (counts + tile - 1) // tile, 0)
    # the GEMM form walks (column tile, row block) entries; entry q runs on XCD q // ceil(n / 8)
    # an expert's tokens split evenly over its tiles, each size rounded up to 32 (the last takes the rest)
    size = [-(-c // n) + 31 & ~31 if n else 0 for c, n in zip(counts, ncol)]
    cols = np.concatenate([np.minimum(z, c - z * np.arange(n)) for c, n, z in zip(counts, ncol, size) if n])
    for name, rows, M in (("gateup", rows_gu, dims.inter), ("down", rows_dn, dims.latent)):
        rb = (M + rows - 1) // rows  # row blocks of each column tile
        work = np.repeat((cols + 15) // 16, rb)  # 16-token column blocks of each entry
        chunk = (work.size + 7) // 8
        per_xcd = np.array([work[x * chunk:(x + 1) * chunk].sum() for x in range(8)], np.float64)
        out[f"{name}_entries"] = int(work.size)
        out[f"{name}_entries_per_xcd"] = int(chunk)
        out[f"{name}_column_blocks_per_xcd_max_over_mean"] = round(float(per_xcd.max() / per_xcd.mean()), 4)
    out["column_tiles"] = int(ncol.sum())
    return out


def bench_graph(dims, xs, pool, row, wts_rot, ws, y, stream, hip_record, steps=64, replays=5):
    """The decode step's kernel launches captured into one HIP graph of `steps` consecutive
    layer calls (tokens from the pool, dense weights rotated as in the eager steps) and
    replayed: the launch gaps between the layer's kernels without the host's launch path.
    Every replay's last output is checked against an eager call on the same token."""
    import torch

    from mxfp4_routed_expert_amd import k3moe
    T = 1
    last = (steps - 1) % pool

    def call(i, out):
        k3moe.k3moe_layer(dims, T, xs.data_ptr() + (i % pool) * row, wts_rot[i % len(wts_rot)], out, None, None,
                          ws, stream=stream)

    y_ref = torch.empty_like(y)
    call(steps - 1, y_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            call(i, y)
    torch.cuda.synchronize()
    ok = True
    with torch.cuda.stream(stream):  # replays run on the stream the events are recorded on
        for _ in range(2):  # replays with eager work and synchronisations between them
            g.replay()
            torch.cuda.synchronize()
            ok = ok and bool(torch.equal(y, y_ref))
            call(0, y)
            torch.cuda.synchronize()
        ms = time_block(lambda i: g.replay(), replays, stream, hip_record) / steps
    torch.cuda.synchronize()
    ok = ok and bool(torch.equal(y, y_ref))
    del g
    log(f"decode T=1 from a HIP graph of {steps} layer steps: {ms * 1e3:.1f} us/step (replays match eager: {ok})")
    return {"us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(1.0 / (ms * 1e-3), 1),
            "steps_per_graph": steps, "replays": replays, "matches_eager": ok, "token_of_last_step": last}


def bench_prefill(args, dims, wts, x, bias_dev, stream, hip_record, what):
    """One prefill workload (x already on the device): ms per step, per-kernel us of a warm
    profiled call, the routing's load balance, algorithmic TFLOP/s."""
    import torch

    from mxfp4_routed_expert_amd import device, k3moe
    T = x.shape[0]
    y = torch.empty((T, dims.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device="cuda")
    ws = device.workspace(dims, T)
    w = wts
    if bias_dev is not None:
        w = type(wts).from_buffer_copy(wts)
        w.bias = bias_dev.data_ptr()

    def step(i):
        k3moe.k3moe_layer(dims, T, x, w, y, idx, None, ws, stream=stream)

    for i in range(2):
        step(i)
    ms = time_block(step, args.prefill_steps, stream, hip_record)
    kern = profiled_kernels(lambda i, ev: k3moe.k3moe_layer_profiled(dims, T, x, w, y, idx, None, ws, ev,
                                                                     stream=stream), 2)
    alg = algorithmic(dims, T, dims.n_experts)
    tf = alg["flops"] / (ms * 1e-3) / 1e12
    ex_us = kern.get("expert_gateup_situ", 0.0) + kern.get("expert_down", 0.0)
    ex_tf = alg["expert_flops"] / (ex_us * 1e-6) / 1e12 if ex_us > 0 else None
    out = {"T": T, "ms_per_step": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
           "algorithmic_TFLOPs": round(tf, 2), "bf16_peak_frac": round(tf / BF16_PEAK_TFLOPS, 4),
           "algorithmic_flops": alg["flops"], "expert_TFLOPs": round(ex_tf, 2) if ex_tf else None,
           "kernel_us": kern, "steps": args.prefill_steps}
    ids = idx.cpu().numpy()
    del y, idx, ws
    torch.cuda.empty_cache()
    log(f"{what}: {ms:.2f} ms/step, {tf:.1f} TFLOP/s algorithmic; per-kernel us: "
        + ", ".join(f"{n} {v:.0f}" for n, v in kern.items()))
    return out, ids


def cpu_baseline(dims, dense, host_blobs, lay, tokens_1, tokens_n):
    """The oracle (plain C, fp64 sums) on K3-shape decode tokens on the host's cores: one
    thread, then OpenMP over tokens on every core of this process's CPU share (at most
    16, the GPU machine's share per GPU)."""
    import k3gen
    import oracle
    ex = oracle.ExpertSet(host_blobs, lay.blob_bytes, lay.offsets)
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    ncores = max(1, min(16, ncores))
    res = {}
    for name, nthreads, n in (("single_thread", 1, tokens_1), ("all_cores", ncores, tokens_n)):
        x = k3gen.gen_x(dims, 1, n)
        c0 = time.perf_counter()
        oracle.layer(dims, x, dense, ex, nthreads=nthreads)
        cs = time.perf_counter() - c0
        res[name] = {"value": round(n / cs, 3), "unit": "tokens/s", "cores": nthreads,
                     "sample": f"{n} K3-shape decode tokens, {cs:.1f} s wall"}
        log(f"cpu oracle: {n / cs:.2f} tokens/s on {nthreads} thread(s)")
    top = dict(res["all_cores"])
    top.update({"kind": "oracle", "sample": top["sample"] + " (OpenMP over tokens); single_thread: "
                + res["single_thread"]["sample"], "single_thread": res["single_thread"]})
    return top


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true", help="skip both prefill workloads")
    ap.add_argument("--no-skewed", action="store_true", help="skip the skewed T = 8192 prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batch-sweep", type=lambda v: [int(t) for t in v.split(",") if t], default=[8, 64, 256],
                    help="also time the layer at these batch sizes (comma list; empty to skip)")
    ap.add_argument("--topp", type=float, default=0.9,
                    help="also time decode with the top-p tail drop at this p (0 = skip); an approximation, "
                         "reported beside the exact layer, never as the headline")
    ap.add_argument("--no-idot", action="store_true",
                    help="skip timing the int8-activation expert variant (an approximation, never the headline)")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the shared-expert measurement (a call of its own, after the layer)")
    ap.add_argument("--no-graph", action="store_true", help="skip the decode steps replayed from a HIP graph")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="oracle tokens on all cores")
    ap.add_argument("--cpu-tokens-1", type=int, default=4, help="oracle tokens on one thread")
    ap.add_argument("--dense-copies", type=int, default=4,
                    help="copies of the dense weights (router, projections) the decode steps rotate "
                         "over, so no step finds them still cached in the MALL from the step before")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a known-size "
                         "kernel for scaling hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the layer is built and timed on a single MI355X; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import k3gen
    from mxfp4_routed_expert_amd import device, k3moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dims = k3gen.K3
    lay = k3gen.ExpertLayout(dims)
    B = lay.blob_bytes

    t0 = time.time()
    dense = k3gen.gen_dense(dims, 1)
    host_blobs = None if args.no_cpu_baseline else np.empty(dims.n_experts * B, np.uint8)

    def chunks():
        for e0 in range(0, dims.n_experts, 32):
            e1 = min(dims.n_experts, e0 + 32)
            out = host_blobs[e0 * B:e1 * B] if host_blobs is not None else None
            yield e0, k3gen.gen_experts(dims, 1, e0, e1, out=out)
    dev = device.upload_layer(dims, dense, chunks(), B, lay.offsets)
    torch.cuda.synchronize()
    log(f"layer generated and uploaded in {time.time() - t0:.1f} s")

    stream = torch.cuda.Stream()
    wts = dev.weights_struct()
    # Decode steps rotate over copies of the dense weights (4 x 128 MB by default) on top of
    # the pool of tokens, so each step's dense weights and experts come from HBM.
    copies = [dev]
    for _ in range(max(1, args.dense_copies) - 1):
        copies.append(device.DeviceLayer(dims=dims, w_router=dev.w_router.clone(), bias=dev.bias.clone(),
                                         w_down=dev.w_down.clone(), w_up=dev.w_up.clone(),
                                         norm_w=dev.norm_w.clone(), experts=dev.experts,
                                         blob_bytes=dev.blob_bytes, offsets=dev.offsets,
                                         gemm_scales=dev.gemm_scales))
        copies[-1].prepare_router_planes()  # of this copy's own router weights
    wts_rot = [c.weights_struct() for c in copies]
    hip_record = ctypes.CDLL("libamdhip64.so").hipEventRecord
    hip_record.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes device to device")
        del src, dst

    # ---------------------------------------------------------------- decode, T = 1
    T = 1
    pool = 64
    xs = torch.from_numpy(k3gen.gen_x(dims, 1, pool).view(np.int16)).cuda()
    y = torch.empty((T, dims.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((pool, dims.topk), dtype=torch.int32, device="cuda")
    tw = torch.empty((pool, dims.topk), dtype=torch.float32, device="cuda")
    ws = device.workspace(dims, T)
    row = dims.hidden * 2

    def step(i):
        j = i % pool
        k3moe.k3moe_layer(dims, T, xs.data_ptr() + j * row, wts_rot[i % len(wts_rot)], y, idx[j], tw[j], ws,
                          stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ms_step = time_block(step, args.steps, stream, hip_record)
    wall = time.perf_counter() - w0
    log(f"decode T=1: {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us/step)")
    # the same kind of steps, each between its own pair of events
    each = np.array(time_each(step, max(20, min(args.steps, 200)), stream, hip_record)) * 1e3
    log(f"decode T=1 per step: median {np.median(each):.1f} us, min {each.min():.1f} us")

    # per-kernel event marks over the same kind of steps
    nprof = min(args.steps, 100)
    kern_us = profiled_kernels(
        lambda i, ev: k3moe.k3moe_layer_profiled(dims, T, xs.data_ptr() + (i % pool) * row, wts_rot[i % len(wts_rot)],
                                                 y, idx[i % pool], tw[i % pool], ws, ev, stream=stream), nprof)
    log("per-kernel us: " + ", ".join(f"{n} {v:.1f}" for n, v in kern_us.items()))

    alg = algorithmic(dims, T, dims.topk)
    layer_gbs = alg["layer_bytes"] / (ms_step * 1e-3) / 1e9
    # the one-token gate/up launch also selects the experts (step name topk_expert_gateup_situ)
    dom = max((n for n in kern_us if n.endswith(("expert_gateup_situ", "expert_down"))),
              key=lambda n: kern_us[n])
    dom_bytes = alg["gateup_bytes"] if dom.endswith("expert_gateup_situ") else alg["down_bytes"]
    dom_gbs = dom_bytes / (kern_us[dom] * 1e-6) / 1e9
    traffic = traffic_from_profile(dom)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch", "algorithmic_bytes": dom_bytes,
                "traffic_over_algorithmic": round(traffic / dom_bytes, 4) if traffic else None,
                "layer_achieved": round(layer_gbs, 1), "layer_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                "layer_bytes": alg["layer_bytes"], "kernel_us": kern_us}
    decode_steps = {"us_mean_block": round(ms_step * 1e3, 2), "us_median": round(float(np.median(each)), 2),
                    "us_min": round(float(each.min()), 2), "us_max": round(float(each.max()), 2),
                    "n_each": int(each.size)}
    graph = None if args.no_graph else bench_graph(dims, xs, pool, row, wts_rot, ws, y, stream, hip_record)

    # ---------------------------------------------------------------- prefill, T = 4096 and skewed T = 8192
    prefill = skewed = None
    if not args.no_prefill:
        xp = torch.from_numpy(k3gen.gen_x(dims, 3, 4096).view(np.int16)).cuda()
        prefill, ids = bench_prefill(args, dims, wts, xp, None, stream, hip_record, "prefill T=4096")
        prefill["routing"] = routing_stats(dims, ids)
        del xp
        if not args.no_skewed:
            with open(os.path.join(ROOT, "tests", "golden", "skew_bias.json")) as f:
                sp = json.load(f)
            sbias = k3gen.skew_bias(dense["bias"], sp["beta"], sp["tail_offset"], sp["hot_every"], sp["tail_from"])
            bias_dev = torch.from_numpy(sbias).cuda()
            xk = torch.from_numpy(k3gen.gen_x(dims, 4, 8192).view(np.int16)).cuda()
            skewed, ids = bench_prefill(args, dims, wts, xk, bias_dev, stream, hip_record,
                                        "skewed prefill T=8192")
            hot = (np.arange(dims.n_experts) % sp["hot_every"]) == 0
            skewed["routing"] = routing_stats(dims, ids, hot)
            del xk, bias_dev
        # MFMA utilisation of the expert GEMMs from the committed counter summary of this
        # same command's prefill (null once the kernel sources differ from the counted ones)
        for obj, tag in ((prefill, "T4096"), (skewed, "T8192")):
            if obj is None:
                continue
            util = {k: figures_from_profile("expert_gemm_prefill_counters.txt", "mfma_util", f"{tag}:{k}")
                    for k in ("expert_gateup_situ", "expert_down")}
            obj["mfma_util"] = util if any(v is not None for v in util.values()) else None
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- small batches
    sweep = {}
    for Tb in args.batch_sweep:
        xb = torch.from_numpy(k3gen.gen_x(dims, 7, Tb).view(np.int16)).cuda()
        yb = torch.empty((Tb, dims.hidden), dtype=torch.float32, device="cuda")
        ib = torch.empty((Tb, dims.topk), dtype=torch.int32, device="cuda")
        wsb = device.workspace(dims, Tb)

        def step_b(i):
            k3moe.k3moe_layer(dims, Tb, xb, wts_rot[i % len(wts_rot)], yb, ib, None, wsb, stream=stream)

        for i in range(3):
            step_b(i)
        msb = time_block(step_b, 10, stream, hip_record)
        ids = ib.cpu().numpy()
        nd = int(np.unique(ids[ids >= 0]).size)
        algb = algorithmic(dims, Tb, nd)
        gbs = algb["layer_bytes"] / (msb * 1e-3) / 1e9
        sweep[str(Tb)] = {"us_per_step": round(msb * 1e3, 1), "tokens_per_s": round(Tb / (msb * 1e-3), 1),
                          "distinct_experts": nd, "algorithmic_bytes": algb["layer_bytes"],
                          "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del xb, yb, ib, wsb
    if sweep:
        log("layer at small batches: " + ", ".join(
            f"T={k} {v['us_per_step']} us ({v['distinct_experts']} experts, {v['GBs']:.0f} GB/s)"
            for k, v in sweep.items()))

    # ---------------------------------------------------------------- top-p tail drop, T = 1
    topp = None
    if args.topp > 0:
        import dataclasses
        dp = dataclasses.replace(dims, topp=args.topp)

        def step_p(i):
            j = i % pool
            k3moe.k3moe_layer(dp, T, xs.data_ptr() + j * row, wts_rot[i % len(wts_rot)], y, idx[j], tw[j], ws,
                              stream=stream)

        for i in range(args.warmup):
            step_p(i)
        ms_p = time_block(step_p, args.steps, stream, hip_record)
        kept = (idx[:min(pool, args.steps)] >= 0).sum(dim=1).float().mean().item()
        topp = {"p": args.topp, "us_per_step": round(ms_p * 1e3, 2), "tokens_per_s": round(1.0 / (ms_p * 1e-3), 1),
                "mean_experts_kept": round(kept, 2), "kind": "approximation (top-p tail drop), not the headline"}
        log(f"decode T=1 with top-p {args.topp}: {ms_p * 1e3:.1f} us/step, {kept:.2f} experts kept on average")

    # ---------------------------------------------------------------- int8 activations, T = 1
    idot = None
    if not args.no_idot:
        import dataclasses
        di = dataclasses.replace(dims, idot=1)

        def step_i(i):
            j = i % pool
            k3moe.k3moe_layer(di, T, xs.data_ptr() + j * row, wts_rot[i % len(wts_rot)], y, idx[j], tw[j], ws,
                              stream=stream)

        for i in range(args.warmup):
            step_i(i)
        ms_i = time_block(step_i, args.steps, stream, hip_record)
        idot = {"us_per_step": round(ms_i * 1e3, 2), "tokens_per_s": round(1.0 / (ms_i * 1e-3), 1),
                "kind": "approximation (int8-per-32 expert activations), not the headline"}
        log(f"decode T=1 with int8 activations: {ms_i * 1e3:.1f} us/step")

    # ---------------------------------------------------------------- shared experts
    shared = None
    if not args.no_shared:
        shared = bench_shared(args, dims, stream, xs, pool, row, hip_record)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dims, dense, host_blobs, lay, args.cpu_tokens_1, args.cpu_tokens)

    out = {
        "metric": "LatentMoE layer tokens/s (K3 decode, T=1); HBM GB/s @T=1, TFLOP/s @T=4096, % of MI355X peak",
        "value": round(1.0 / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "K3-shape decode layer T=1: H=7168 L=3584 I=3072 E=896 K=16, "
                               "896 MXFP4 experts resident (15.7 GB), 64-token pool, dense weights "
                               f"rotated over {len(wts_rot)} copies", "T": T, "global_batch": T,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "decode_steps": decode_steps,
        "decode_graph": graph,
        "prefill": prefill,
        "skewed_prefill": skewed,
        "batch_sweep": sweep or None,
        "shared_experts": shared,
        "topp_decode": topp,
        "idot_decode": idot,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
