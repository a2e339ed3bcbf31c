#!/usr/bin/env python3
"""Benchmark of the local MoE expert layer on one MI355X.

One step = the whole hot path over one batch of synthetic input resident in HBM:
routing metadata from topk_idx/topk_weights [N,K], the forward (gathered
up-projection + SwiGLU, down projection, weighted combine), and the backward
(dx, dW_up, dW_down, d_topk_weights). The default workload is one EP8 rank's
share of a 256-expert top-8 layer: N=16384 received rows, H=2048, I=512, E=32
local experts, K=8 (the Qwen3.6 serving-script notes: 256 experts x top-8 at
16384 tokens; GitHub issue #68: EP8 with DeepEP non-expand inputs).

Prints one JSON line: throughput in TFLOP/s over valid pairs (18*P*H*I per
forward+backward step; the median of per-step event times after 10 warm-up steps),
the routing-metadata build time and its fraction of HBM bandwidth, the dominant
kernel against its roofline (timed with HIP events on its own stream through the
library's kernel-timing hook), the CPU oracle timed on a bounded sample of the same
workload on this host, and under "workloads" a few steps of each other benchmarked
layer: the DeepSeek-V3-style and long-prefill rank shares (fwd+bwd) and decode
(forward, weight-streaming GB/s).
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE expert fwd+bwd TFLOP/s and % bf16 MFMA peak; metadata build µs, "
          "% HBM BW")
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E

# algorithmic flops of each GEMM kernel per launch, in units of P*H*I
GEMM_FLOPS = {"up_swiglu": 4, "down": 2, "down_bwd": 2, "wgrad_down": 2, "up_bwd": 4,
              "wgrad_up": 4}
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)  # flop/byte where the rooflines meet


def gemm_bytes(kernel, N, H, I, P, active):
    """Algorithmic HBM bytes of one launch (bf16): each operand and result once; the
    weights of the experts that have rows (`active` of them)."""
    w_up, w_down = active * H * 2 * I * 2, active * I * H * 2
    return {
        "up_swiglu": 2 * P * H + w_up + 2 * P * 2 * I + 2 * P * I,   # x rows, W_up, h, a
        "down": 2 * P * I + w_down + 2 * P * H,                      # a, W_down, y
        "down_bwd": 2 * P * H + w_down + 2 * P * 2 * I * 2 + 2 * P * I,  # dout rows, W_down, h, dh, w*a
        "wgrad_down": 2 * P * I + 2 * P * H + w_down,                # w*a, dout rows, dW_down
        "up_bwd": 2 * P * 2 * I + w_up + 2 * P * H,                  # dh, W_up, dxg
        "wgrad_up": 2 * P * H + 2 * P * 2 * I + w_up,                # x rows, dh, dW_up
    }[kernel]


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "token_routing_grouped_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("bytes_per_launch")


class TimingEvent:
    """A HIP event for timing only (hipEventDisableSystemFence): recording it does not
    write back and invalidate the caches, which with default events opened a ~6 us gap
    before and after the bracketed kernel. Same interface as torch.cuda.Event for
    moe_time_kernel (cuda_event) and for reading (elapsed_time, in ms)."""
    _hip = None

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            try:
                TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
            except OSError:
                TimingEvent._hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
        self._ct = ctypes
        h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self, stream_ptr: int) -> None:
        rc = TimingEvent._hip.hipEventRecord(self._ct.c_void_p(self.cuda_event),
                                             self._ct.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float(0.0)
        rc = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self._ct.c_void_p(self.cuda_event),
                                                  self._ct.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if TimingEvent._hip is not None and getattr(self, "cuda_event", None):
                TimingEvent._hip.hipEventDestroy(self._ct.c_void_p(self.cuda_event))
        except Exception:  # interpreter shutdown
            pass


def cpu_baseline(d, backward: bool, target_s: float):
    """The oracle (fp64, OpenMP) on the first tokens of the workload: metadata,
    forward and (if the workload has it) backward, on full tensors of that sample."""
    import numpy as np

    import oracle

    f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wu, wd = f64(d["w_up"]), f64(d["w_down"])
    idx, w = d["topk_idx"], d["topk_weights"]
    H, I, E = d["H"], d["I"], d["E"]
    valid = (idx >= 0).sum(axis=1)
    csum = np.cumsum(valid)
    mult = (18 if backward else 6) * H * I

    def run(pairs):
        n = int(np.searchsorted(csum, pairs)) + 1
        n = min(n, idx.shape[0])
        t0 = time.perf_counter()
        m = oracle.build_metadata(idx[:n], w[:n], E)
        x = f64(d["x"][:n])
        f = oracle.forward(x, wu, wd, m)
        if backward:
            oracle.backward(x, wu, wd, f64(d["dout"][:n]), m, f)
        return n, m["P"], time.perf_counter() - t0

    n, P, t = run(512)  # calibration
    rate = P * mult / max(t, 1e-6)
    want = int(min(csum[-1], max(512, target_s * rate / mult)))
    n, P, t = run(want)
    t0 = time.perf_counter()
    oracle.build_metadata(idx, w, E)
    t_meta = time.perf_counter() - t0
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {
        "value": P * mult / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
        "kind": "oracle", "cpu_model": cpu_model,
        "sample": (f"first {n} of {idx.shape[0]} rows ({P} pairs): metadata + forward"
                   f"{' + backward' if backward else ''} in fp64, {t:.1f} s"),
        "metadata_us_full_workload": t_meta * 1e6,
    }


def metadata_sweep(moe, synth, torch, np):
    """Metadata build alone over N = 2^14..2^20 at K=8, E=64: device time of 20 builds
    captured in one HIP graph, and the algorithmic bytes over that time."""
    dev = torch.device("cuda:0")
    K, E, reps = 8, 64, 20
    rows = []
    for logn in range(14, 21):
        N = 1 << logn
        idx_np = synth.routing_uniform(N, E, K, p_invalid=0.2, min_valid=0, seed=logn)
        w_np = synth.make_topk_weights(idx_np, logn)
        P = int((idx_np >= 0).sum())
        idx = torch.from_numpy(idx_np).to(dev)
        w = torch.from_numpy(w_np).to(dev)
        meta = moe.Metadata(N, K, E, P, device=dev)
        ws = torch.empty(max(1, moe.moe_build_metadata_workspace(N, K, E)), dtype=torch.uint8,
                         device=dev)
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            moe.moe_build_metadata(idx, w, meta, workspace=ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            for _ in range(reps):
                moe.moe_build_metadata(idx, w, meta, workspace=ws)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        assert int(meta.status.item()) == 0
        us = 1e3 * e0.elapsed_time(e1) / reps
        nbytes = 8 * N * K + 16 * P + 4 * (N + 1) + 4 * E + 4 * (E + 1)
        rows.append({"N": N, "P": P, "us": round(us, 2), "bytes": nbytes,
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)})
        print(json.dumps(rows[-1]), flush=True)
    print(json.dumps({"metric": "metadata build time and HBM fraction, K=8 E=64",
                      "unit": "us", "sweep": rows}), flush=True)


def token_sweep(moe, synth, torch, np, stream, steps, warmup):
    """The default workload's step (H 2048, I 512, 32 local experts of 256 global, top-8,
    the same routing recipe) at other token counts per rank, N = 2^10 .. 2^16: where tile
    quantisation, launch latency and the fixed per-call work begin to weigh."""
    base = synth.CONFIGS["qwen3_rank"]
    rows = []
    for logn in range(10, 17):
        name = f"qwen3_rank_n{1 << logn}"
        synth.CONFIGS[name] = dict(base, N=1 << logn)
        r, _ = measure(moe, synth, torch, np, name, 0, steps, warmup, 0, stream)
        r.pop("_handles", None)
        row = {"N": r["N"], "P": r["P"], "ms_per_step": r["ms_per_step"],
               "TFLOPs": r["TFLOPs"], "mfma_frac": r["mfma_frac"],
               "dominant": r["roofline"]["kernel"], "dominant_bound": r["roofline"]["bound"],
               "dominant_achieved": r["roofline"]["achieved"],
               "dominant_unit": r["roofline"]["unit"], "dominant_frac": r["roofline"]["frac"],
               "kernels_us": r["kernels_us"]}
        rows.append(row)
        print(json.dumps(row), flush=True)
    print(json.dumps({"metric": "fwd+bwd step over tokens per rank (H 2048, I 512, E 32, K 8)",
                      "unit": "TFLOP/s", "sweep": rows}), flush=True)


def router_timing(moe, synth, torch, np, N=32768, E=128, K=8, reps=20):
    """moe_route (top-K + weights + aux loss + the metadata) alone, at the routing
    example of the Hysen Labs page (32768 tokens, 128 experts, top-8, fp32 logits):
    device time of reps calls captured in one HIP graph, algorithmic bytes over it."""
    dev = torch.device("cuda:0")
    lg = torch.from_numpy(synth.router_logits(N, E, seed=1)).to(dev)
    meta = moe.Metadata(N, K, E, N * K, device=dev)
    idx = torch.empty(N, K, dtype=torch.int32, device=dev)
    w = torch.empty(N, K, dtype=torch.float32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, moe.moe_route_workspace(N, K, E)), dtype=torch.uint8, device=dev)

    def call():
        moe.moe_route(lg, meta, mode=moe.MOE_ROUTE_TOPK_SOFTMAX, renormalize=True, topk_idx=idx,
                      topk_weights=w, aux_loss=aux, workspace=ws)

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for _ in range(reps):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / reps
    P = N * K
    # logits read; topk_idx/weights written then re-read by the scatter; metadata written
    nbytes = 4 * N * E + 8 * N * K * 2 + 16 * P + 4 * (N + 1) + 4 * E + 4 * (E + 1)
    return {"N": N, "E": E, "K": K, "mode": "topk_of_softmax+renorm", "us": round(us, 2),
            "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}


def step_bytes_decode(d, P, active):
    """Algorithmic HBM bytes of one forward (bf16): the active experts' weights, the
    gathered x rows, h and a written, a re-read, y written and re-read, out written."""
    N, H, I = d["N"], d["H"], d["I"]
    return (active * 6 * H * I + 2 * P * H + 2 * P * 2 * I + 2 * 2 * P * I + 2 * 2 * P * H
            + 2 * N * H)


def measure(moe, synth, torch, np, name, seed, steps, warmup, cold_reps, stream):
    """Times one workload: warm-up steps, the per-kernel durations (to name the dominant
    kernel), then `steps` steps between a synchronisation on each side with an event
    after every step (median and mean per step) and the dominant kernel bracketed by
    events on its stream, then single cold steps. Returns (result dict, inputs)."""
    cfg = synth.CONFIGS[name]
    backward = cfg["backward"]
    d = synth.make_inputs(name, seed, dout=backward)
    N, H, I, E, K = d["N"], d["H"], d["I"], d["E"], d["K"]
    P = int((d["topk_idx"] >= 0).sum())
    dev = torch.device("cuda:0")

    def t(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, w_up, w_down = t(d["x"]), t(d["w_up"]), t(d["w_down"])
    dout = t(d["dout"]) if backward else None
    idx = torch.from_numpy(d["topk_idx"]).to(dev)
    w = torch.from_numpy(d["topk_weights"]).to(dev)
    # capacity = P, known on the host as DeepEP's handle knows total_pairs
    meta = moe.Metadata(N, K, E, P, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    ws_meta = torch.empty(max(1, moe.moe_build_metadata_workspace(N, K, E)), **u8)
    ws_fwd = torch.empty(max(1, moe.moe_expert_forward_workspace(meta, H, I)), **u8)
    ws_bwd = (torch.empty(max(1, moe.moe_expert_backward_workspace(meta, H, I)), **u8)
              if backward else None)
    out = torch.empty(N, H, dtype=torch.bfloat16, device=dev)
    h_save = torch.empty(P, 2 * I, dtype=torch.bfloat16, device=dev) if backward else None
    if backward:
        dx = torch.empty_like(x)
        dw_up = torch.empty_like(w_up)
        dw_down = torch.empty_like(w_down)
        dtw = torch.empty(N, K, dtype=torch.float32, device=dev)

    def build():
        moe.moe_build_metadata(idx, w, meta, workspace=ws_meta)

    def step():
        build()
        moe.moe_expert_forward(meta, x, w_up, w_down, out, h_save=h_save, workspace=ws_fwd)
        if backward:
            moe.moe_expert_backward(meta, idx, x, w_up, w_down, h_save, dout, dx, dw_up,
                                    dw_down, dtw, workspace=ws_bwd)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    status = int(meta.status.item())
    assert status == 0, f"device status {status}"
    assert torch.isfinite(out.float()).all()

    # per-kernel durations (3 launches each) to name the dominant kernel
    # the kernels one step launches (the router is timed on its own)
    step_kernels = [k for k in moe.KERNELS if not k.startswith("route")]
    kernels = step_kernels if backward else step_kernels[:step_kernels.index("combine") + 1]
    kernel_us = {}
    for k in kernels:
        ev = [TimingEvent() for _ in range(6)]
        moe.moe_time_kernel(k, ev)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        if moe.moe_time_kernel(k, None) < 3:
            continue  # not launched at this size
        kernel_us[k] = 1e3 * sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(3)) / 3
    gemms = {k: v for k, v in kernel_us.items() if k in GEMM_FLOPS}
    dominant = max(gemms, key=gemms.get)

    # timed region: `steps` steps, an event after each, the dominant kernel bracketed
    ev = [TimingEvent() for _ in range(2 * steps)]
    marks = [TimingEvent() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    moe.moe_time_kernel(dominant, ev)
    wall0 = time.perf_counter()
    stream_ptr = stream.cuda_stream
    marks[0].record(stream_ptr)
    for i in range(steps):
        step()
        marks[i + 1].record(stream_ptr)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    nrec = moe.moe_time_kernel(dominant, None)
    assert nrec == steps, nrec
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    ms_med = per_step[len(per_step) // 2] if steps % 2 else \
        0.5 * (per_step[steps // 2 - 1] + per_step[steps // 2])
    ms_mean = marks[0].elapsed_time(marks[steps]) / steps
    dom_times = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    dom_ms = sum(dom_times) / steps
    assert int(meta.status.item()) == 0

    # cold: each single step follows a 1 GiB fill that evicts L2 and the 256 MB MALL
    cold = []
    if cold_reps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for _ in range(cold_reps):
            flush.zero_()
            marks[0].record(stream_ptr)
            step()
            marks[1].record(stream_ptr)
            torch.cuda.synchronize()
            cold.append(marks[0].elapsed_time(marks[1]))
        del flush
        cold.sort()

    flops_step = (18 if backward else 6) * P * H * I
    tflops = flops_step / (ms_med * 1e-3) / 1e12
    dom_flops = GEMM_FLOPS[dominant] * P * H * I
    dom_tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    active = int((np.bincount(d["topk_idx"][d["topk_idx"] >= 0].ravel(), minlength=E) > 0).sum())
    dom_bytes = gemm_bytes(dominant, N, H, I, P, active)
    # the roofline that bounds the kernel: HBM below the ridge intensity (decode), else MFMA
    hbm_bound = dom_flops / dom_bytes < RIDGE
    if hbm_bound:
        roof = {"kernel": dominant, "bound": "hbm",
                "achieved": round(dom_bytes / (dom_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(dom_bytes / (dom_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    else:
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(dom_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4)}
    roof.update({"traffic": counted_traffic(dominant, name), "avg_us": round(dom_ms * 1e3, 2),
                 "median_us": round(dom_times[len(dom_times) // 2] * 1e3, 2),
                 "flops_per_launch": dom_flops, "bytes_per_launch": dom_bytes,
                 "intensity_flop_per_byte": round(dom_flops / dom_bytes, 1)})
    res = {
        "N": N, "H": H, "I": I, "E": E, "K": K, "P": P, "seed": d["seed"],
        "step": "metadata + forward" + (" + backward" if backward else ""),
        "flops_per_step": flops_step, "ms_per_step": round(ms_med, 4),
        "mean_ms_per_step": round(ms_mean, 4), "TFLOPs": round(tflops, 2),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "cold": ({"ms_per_step": round(cold[len(cold) // 2], 4),
                  "TFLOPs": round(flops_step / (cold[len(cold) // 2] * 1e-3) / 1e12, 2),
                  "reps": len(cold)} if cold else None),
        "kernels_us": {k: round(v, 1) for k, v in kernel_us.items()},
        "roofline": roof, "wall_s_timed": round(wall, 4), "steps": steps, "warmup": warmup,
    }
    if not backward:  # a forward at decode size streams the active experts' weights
        nb = step_bytes_decode(d, P, active)
        res.update({"us_per_step": round(ms_med * 1e3, 2), "active_experts": active,
                    "bytes_per_step": nb,
                    "GBps": round(nb / (ms_med * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nb / (ms_med * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)})
    res["_handles"] = (idx, w, meta, ws_meta)
    return res, d


def metadata_alone(torch, moe, handles, stream, nm=50):
    """Metadata build alone: device time of nm builds captured in one HIP graph (the
    build never syncs with the host, so it captures) and replayed between events; and
    the same nm calls issued from Python (bounded by host launch overhead)."""
    idx, w, meta, ws_meta = handles

    def build():
        moe.moe_build_metadata(idx, w, meta, workspace=ws_meta)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    with torch.cuda.stream(cap_stream):
        build()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap_stream):
        for _ in range(nm):
            build()
    graph.replay()
    torch.cuda.synchronize()
    reps = []
    for _ in range(5):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(1e3 * e0.elapsed_time(e1) / nm)
    reps.sort()
    e0.record(stream)
    for _ in range(nm):
        build()
    e1.record(stream)
    torch.cuda.synchronize()
    return reps[len(reps) // 2], 1e3 * e0.elapsed_time(e1) / nm


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_rank")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only --workload (by default the line also carries a few steps "
                         "of each other benchmarked workload, and of the default workload at "
                         "1024 and 4096 tokens)")
    ap.add_argument("--other-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="single steps timed after a 1 GiB fill evicts L2 and the MALL")
    ap.add_argument("--metadata-sweep", action="store_true",
                    help="instead of the benchmark, time the metadata build alone for "
                         "N = 2^14 .. 2^20 rows at K=8, E=64 (uniform routing, 20%% -1 slots)")
    ap.add_argument("--token-sweep", action="store_true",
                    help="instead of the benchmark, time the default workload's step at "
                         "N = 2^10 .. 2^16 tokens (the --steps and --warmup given)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB "
                         "(reference kernel for scaling HBM traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one rank's local expert layer on one GPU: --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_mib:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        e0.record()
        for _ in range(3):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        nb = args.copy_mib << 20
        # a copy moves its size twice (read and write)
        print(json.dumps({"copy_bytes": nb, "launches": 4, "ms_per_copy": round(ms, 4),
                          "GBps_read_plus_write": round(2 * nb / (ms * 1e-3) / 1e9, 1)}))
        return

    import synth
    import token_routing_grouped_amd as moe

    if args.metadata_sweep:
        metadata_sweep(moe, synth, torch, np)
        return
    if args.token_sweep:
        torch.cuda.set_device(torch.device("cuda:0"))
        token_sweep(moe, synth, torch, np, torch.cuda.current_stream(), args.steps, args.warmup)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    r, d = measure(moe, synth, torch, np, args.workload, args.seed, args.steps, args.warmup,
                   args.cold_reps, stream)
    meta_us, meta_eager_us = metadata_alone(torch, moe, r.pop("_handles"), stream)
    N, E, K, P = r["N"], r["E"], r["K"], r["P"]
    meta_bytes = 8 * N * K + 16 * P + 4 * (N + 1) + 4 * E + 4 * (E + 1)
    backward = synth.CONFIGS[args.workload]["backward"]
    res = {
        "metric": METRIC,
        "value": r["TFLOPs"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "N": N, "H": r["H"], "I": r["I"], "E": E, "K": K,
                   "P": P, "seed": r["seed"], "step": r["step"],
                   "flops_per_step": r["flops_per_step"]},
        "timing": "median of per-step event times over the timed steps",
        "mean_ms_per_step": r["mean_ms_per_step"],
        "mfma_frac": r["mfma_frac"],
        "cold": r["cold"],
        "metadata": {"us": round(meta_us, 2), "eager_us": round(meta_eager_us, 2),
                     "bytes": meta_bytes,
                     "GBps": round(meta_bytes / (meta_us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(meta_bytes / (meta_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)},
        "kernels_us": r["kernels_us"],
        "roofline": r["roofline"],
        "wall_s_timed": r["wall_s_timed"],
    }
    del r
    torch.cuda.empty_cache()
    res["router"] = router_timing(moe, synth, torch, np)
    if not args.no_other_workloads:
        others = {}
        for name in ("dsv3_rank", "long_prefill", "decode"):
            if name == args.workload:
                continue
            print(f"bench: {name}", file=sys.stderr, flush=True)
            ro, _ = measure(moe, synth, torch, np, name, args.seed, args.other_steps, 3, 0,
                            stream)
            handles = ro.pop("_handles")
            ro.pop("cold")
            if not synth.CONFIGS[name]["backward"]:
                ro["metadata_us"] = round(metadata_alone(torch, moe, handles, stream)[0], 2)
            del handles
            others[name] = ro
            torch.cuda.empty_cache()
        res["workloads"] = others
        # the default workload at small token counts per rank (where its GEMMs take the
        # 128x128 tiles): step time and the longest GEMM against its roofline
        small = []
        for n in (1024, 4096):
            name = f"qwen3_rank_n{n}"
            synth.CONFIGS[name] = dict(synth.CONFIGS["qwen3_rank"], N=n)
            print(f"bench: {name}", file=sys.stderr, flush=True)
            ro, _ = measure(moe, synth, torch, np, name, args.seed, args.other_steps, 3, 0,
                            stream)
            ro.pop("_handles")
            small.append({"N": n, "P": ro["P"], "ms_per_step": ro["ms_per_step"],
                          "TFLOPs": ro["TFLOPs"], "longest_gemm": ro["roofline"]["kernel"],
                          "bound": ro["roofline"]["bound"],
                          "achieved": ro["roofline"]["achieved"],
                          "unit": ro["roofline"]["unit"], "frac": ro["roofline"]["frac"]})
            torch.cuda.empty_cache()
        res["qwen3_rank_small_n"] = small
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, backward, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
