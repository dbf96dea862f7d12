#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer (MXFP4 experts) on one MI355X.

One step = one call of moe_layer_forward over one batch: router, top-8,
grouping, gate/up + SwiGLU, down projection and weighted combine.  The headline
workload is decode at batch 1 on the MiMo-shaped layer (hidden 4096,
intermediate 2048, 256 experts, top-8, 3,422,552,064 bytes of MXFP4 experts).

Cache protocol: the 256 MB last-level cache could hold a decode step's
111 MB working set, so steps cycle through --layers device copies of the layer
and every step takes a fresh token; a reused expert is then never still cached.

Prints ONE JSON line (rank 0): metric/value (tokens/s), roofline of the
dominant kernel, the CPU oracle timed on a bounded sample, and extra workloads
(16-token verify with skewed routing, 2048-token MXFP4 and VQ13R8 prefill)
with their own rooflines.  A kernel's launch duration is measured with two HIP
events on the stream it runs on around `steps` back-to-back launches of it
(moe_layer_replay_stage over the last step's routing, cycling the layer
copies), so it compares directly with a rocprofv3 kernel trace.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA % of peak (1 GPU)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_quantized_moe_gemv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic(kernel: str, src: tuple, launches_units: float):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    if there is none or the kernel's sources (its file and the shared device
    header) changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_sha256") != _src_hash(*src):
        return None
    return d.get("hbm_bytes_per_launch")


def read_probe_gbs(torch, bq, nbytes, n_copies, reps):
    """Plain streaming read (moe_read_probe) of nbytes, cycling n_copies
    device copies so the last-level cache does not serve them: GB/s over
    `reps` back-to-back reads, timed with HIP events on the probe's stream."""
    stride = (nbytes + 255) // 256 * 256
    buf = torch.ones(stride * n_copies, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    bq.read_probe(buf.data_ptr(), nbytes, stride, n_copies, max(4, reps // 10), sink.data_ptr(),
                  st.cuda_stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    bq.read_probe(buf.data_ptr(), nbytes, stride, n_copies, reps, sink.data_ptr(), st.cuda_stream)
    e1.record(st)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del buf
    torch.cuda.empty_cache()
    return round(nbytes / (us * 1e-6) / 1e9, 1), round(us, 3)


def measured_peaks(torch, bq, step_bytes):
    """Attainable peaks on this machine: a device-to-device copy, plain streaming
    reads (of 2 GiB, and of one decode step's footprint over 8 copies), and a
    bf16 GEMM."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    it = 10
    for _ in range(it):
        b.copy_(a)
    torch.cuda.synchronize()
    copy_gbs = 2 * n * it / (time.perf_counter() - t0) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        x @ y
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    it = 20
    for _ in range(it):
        x @ y
    torch.cuda.synchronize()
    tflops = 2 * m ** 3 * it / (time.perf_counter() - t0) / 1e12
    del x, y
    torch.cuda.empty_cache()
    big_gbs, _ = read_probe_gbs(torch, bq, 2 << 30, 1, 20)
    step_gbs, step_us = read_probe_gbs(torch, bq, step_bytes, 8, 400)
    return {"copy_gbs": round(copy_gbs, 1), "read_probe_gbs_2gib": big_gbs,
            "read_probe_gbs_decode_step": step_gbs, "read_probe_decode_step_bytes": step_bytes,
            "read_probe_decode_step_us": step_us, "bf16_matmul_tflops": round(tflops, 1)}


class Bench:
    def __init__(self, args, torch, bq, W):
        self.args, self.torch, self.bq, self.W = args, torch, bq, W
        base = W.DECODE
        log(f"generating the MiMo-shaped MXFP4 layer ({base.packed_bytes} B)")
        t0 = time.perf_counter()
        self.host_layer = W.make_experts(base)
        log(f"  {time.perf_counter() - t0:.1f}s; copying {args.layers} device copies")
        self.input_hashes = {f"{base.name}.packed_experts": W.sha256(self.host_layer),
                             f"{base.name}.router_w": W.sha256(W.make_router(base))}
        self.layers = self._copies(self.host_layer, args.layers)
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()

    def _copies(self, host, n):
        """n device copies of a packed layer, back to back in one allocation:
        (tensor, base pointer, stride in bytes, n)."""
        torch = self.torch
        nb = host.nbytes
        stride = (nb + 255) // 256 * 256
        big = torch.empty(stride * n, dtype=torch.uint8, device="cuda")
        src = torch.from_numpy(host).to("cuda")
        for i in range(n):
            big[i * stride:i * stride + nb].copy_(src)
        del src
        return big, int(big.data_ptr()), stride, n

    def vq_layers(self):
        """--layers device copies of the VQ13R8 layer (2.1 GB each), cycled like the
        MXFP4 copies so that replayed stages do not find the last launch's
        experts in the last-level cache."""
        if not hasattr(self, "_vq"):
            W, torch = self.W, self.torch
            log(f"generating the MiMo-shaped VQ13R8 layer ({W.VQ_PREFILL.packed_bytes} B)")
            host = W.make_experts(W.VQ_PREFILL)
            self._vq = self._copies(host, self.args.layers)
            del host
            torch.cuda.synchronize()
        return self._vq

    def vq13_layers(self):
        """--layers device copies of the VQ13 layer (1.3 GB each), cycled."""
        if not hasattr(self, "_vq13"):
            W, torch = self.W, self.torch
            log(f"generating the MiMo-shaped VQ13 layer ({W.VQ13_DECODE.packed_bytes} B)")
            host = W.make_experts(W.VQ13_DECODE)
            self._vq13 = self._copies(host, self.args.layers)
            del host
            torch.cuda.synchronize()
        return self._vq13

    def graph_steps(self, wl, n_cap=64, reps=40):
        """The step replayed from a captured graph: n_cap forwards (a fresh
        token each, cycling the layer copies) captured once into a graph, the
        graph replayed reps times between two HIP events; microseconds per
        forward."""
        torch, bq, W = self.torch, self.bq, self.W
        T = wl.tokens
        x = W.make_x(wl, tokens=T * n_cap, stream_offset=77)
        xd = torch.from_numpy(x.view("int16")).to("cuda").view(torch.bfloat16).view(n_cap, T,
                                                                                  wl.hidden)
        wr = torch.from_numpy(W.make_router(wl)).to("cuda")
        layer = bq.MoeLayer(wl.hidden, wl.inter, wl.experts, wl.top_k, T, wl.fmt, 0,
                            routing=wl.routing)
        out = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
        _, base, stride, L = self.layers
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm the handle outside the capture
            layer.forward(xd[0], wr, self.layers[0][:stride], out=out, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream().cuda_stream
            for i in range(n_cap):
                rc = layer.forward_raw(int(xd[i].data_ptr()), T, int(wr.data_ptr()),
                                       base + (i % L) * stride, int(out.data_ptr()), st)
                if rc != 0:
                    raise bq.MoeError(rc, "moe_layer_forward (capture)")
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n_cap)
        del g
        layer.close()
        return round(us, 3)

    def run(self, wl, steps, warmup, tokens_per_step, profile=True, layers=None, replay=0,
            path=0, clock_warmup_s=0.0):
        torch, bq, W = self.torch, self.bq, self.W
        T = tokens_per_step
        n_batches = steps + warmup
        # a fresh batch of tokens for every step
        xs = []
        per = 1 if wl.scaled_tokens else max(1, 4096 // T)
        for off in range(0, n_batches, per):
            cnt = min(per, n_batches - off)
            x = W.make_x(wl, tokens=T * cnt, stream_offset=1 + off)
            xs.append(torch.from_numpy(x.view("int16")).to("cuda").view(torch.bfloat16))
        xall = torch.cat(xs).view(n_batches, T, wl.hidden)
        if wl.name == W.DECODE.name:
            self.input_hashes[f"{wl.name}.x_all_steps"] = W.sha256(
                xall.view(torch.int16).cpu().numpy())
        wr = torch.from_numpy(W.make_router(wl)).to("cuda")
        layer = bq.MoeLayer(wl.hidden, wl.inter, wl.experts, wl.top_k, T, wl.fmt, path,
                            routing=wl.routing)
        out = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
        st = self.stream.cuda_stream
        _, base, stride, L = self.layers if layers is None else layers
        xp = [int(xall[i].data_ptr()) for i in range(n_batches)]
        lp = [base + i * stride for i in range(L)]
        wp, op = int(wr.data_ptr()), int(out.data_ptr())

        def loop(i0, n):
            for i in range(i0, i0 + n):
                rc = layer.forward_raw(xp[i], T, wp, lp[i % L], op, st)
                if rc != 0:
                    raise bq.MoeError(rc, "moe_layer_forward")

        if clock_warmup_s > 0:
            # untimed forwards over the warm-up tokens (cycling the layer
            # copies) until the GPU has run for clock_warmup_s, so that the
            # timed steps do not start at an idle clock
            t_end, i = time.perf_counter() + clock_warmup_s, 0
            while time.perf_counter() < t_end:
                for _ in range(64):
                    rc = layer.forward_raw(xp[i % max(1, warmup)], T, wp, lp[i % L], op, st)
                    if rc != 0:
                        raise bq.MoeError(rc, "moe_layer_forward")
                    i += 1
                torch.cuda.synchronize()
        loop(0, warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        loop(warmup, steps)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        res = {"steps": steps, "warmup": warmup, "ms_per_step": elapsed * 1e3 / steps,
               "tokens_per_s": steps * T / elapsed, "path": layer.last_path()}
        # the same steps again with a HIP event between consecutive steps on
        # the forward's stream: the median step interval
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(self.stream)
        for i in range(steps):
            rc = layer.forward_raw(xp[warmup + i], T, wp, lp[(warmup + i) % L], op, st)
            if rc != 0:
                raise bq.MoeError(rc, "moe_layer_forward")
            evs[i + 1].record(self.stream)
        evs[-1].synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        res["event_median_ms_per_step"] = round(per[steps // 2], 5)
        # routing statistics of the last step (distinct experts streamed)
        r = layer.routing()
        counts = r.counts.cpu()
        res["distinct_experts_last_step"] = int((counts > 0).sum())
        if replay:
            # each expert kernel alone: `replay` back-to-back launches of one
            # stage of the last step (cycling the layer copies) between two
            # events on the stream the kernels run on
            res["replay_us"] = {}
            stages = (("router", "gateup", "down") if layer.last_path() == bq.MOE_PATH_DECODE
                      else bq.STAGES)
            for stage in stages:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
                rc = layer.replay_stage_raw(stage, replay, xp[warmup + steps - 1], wp, base,
                                            stride, L, op, st)
                e1.record(self.stream)
                if rc != 0:
                    raise bq.MoeError(rc, "moe_layer_replay_stage")
                e1.synchronize()
                res["replay_us"][stage] = round(e0.elapsed_time(e1) * 1e3 / replay, 3)
        if profile:
            # second pass over the same steps with event pairs around each kernel
            layer.set_profiling(steps)
            loop(warmup, steps)
            torch.cuda.synchronize()
            prof = layer.profile_read()
            layer.set_profiling(0)
            stages = {}
            for name in bq.STAGES:
                v = [p[name] for p in prof if name in p]
                if v:
                    stages[name] = sum(v) / len(v) * 1e3  # microseconds
            res["stage_us"] = {k: round(v, 2) for k, v in stages.items()}
            res["profiled_ms_per_step"] = sum(stages.values()) / 1e3
        layer.close()
        return res


def algorithmic(wl, distinct, T):
    """Algorithmic bytes / flops of the gate/up and down kernels and the whole
    step.  Per expert: MXFP4 gate/up 2*I*H*17/32 bytes and down H*I*17/32
    bytes; VQ13R8 21/64 byte per weight (VQ13 13/64) plus an fp16 gain per row."""
    H, I, k = wl.hidden, wl.inter, wl.top_k
    R = T * k
    if wl.fmt in (W_FMT_VQ, W_FMT_VQ13):
        bits = 21 if wl.fmt == W_FMT_VQ else 13  # index bits per 8-weight vector
        gu_e = 2 * I * H * bits // 64 + 2 * (2 * I)
        dn_e = H * I * bits // 64 + 2 * H
    elif wl.fmt == W_FMT_MXFP4:
        gu_e = 2 * I * H * 17 // 32
        dn_e = H * I * 17 // 32
    else:
        raise ValueError(f"unknown expert format {wl.fmt}")
    gateup_bytes = distinct * gu_e + T * H * 2 + R * I * 4
    down_bytes = distinct * dn_e + R * I * 4 + T * H * 4
    step_bytes = distinct * (gu_e + dn_e) + wl.experts * H * 4 + T * H * 2 + T * H * 4
    flops_gu = 2 * R * 2 * I * H
    flops_dn = 2 * R * H * I
    return dict(gateup_bytes=gateup_bytes, down_bytes=down_bytes, step_bytes=step_bytes,
                gateup_flops=flops_gu, down_flops=flops_dn, step_flops=flops_gu + flops_dn)


W_FMT_MXFP4, W_FMT_VQ, W_FMT_VQ13 = 1, 2, 3


def prefill_report(pre, a):
    pf = a["step_flops"] / (pre["ms_per_step"] * 1e-3) / 1e12
    gu_t = a["gateup_flops"] / (pre["replay_us"]["gateup"] * 1e-6) / 1e12
    dn_t = a["down_flops"] / (pre["replay_us"]["down"] * 1e-6) / 1e12
    return {
        **pre, "step_algorithmic_flops": a["step_flops"],
        "step_algorithmic_bytes": a["step_bytes"],
        "step_mfma_tflops": round(pf, 1), "step_mfma_frac": round(pf / BF16_PEAK_TFLOPS, 4),
        "step_hbm_frac": round(a["step_bytes"] / (pre["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "gateup_mfma_frac": round(gu_t / BF16_PEAK_TFLOPS, 4),
        "down_mfma_frac": round(dn_t / BF16_PEAK_TFLOPS, 4),
    }


def cpu_baseline(host_layer, W, n_tokens, runs):
    """The oracle on `runs` independent batches of n_tokens decode tokens of
    the benchmarked layer: the median rate."""
    import oracle

    wl = W.DECODE
    wr = W.make_router(wl)
    rates, secs = [], []
    for r in range(runs):
        x = W.make_x(wl, tokens=n_tokens, stream_offset=999 + r)
        t0 = time.perf_counter()
        oracle.moe_forward(wl.fmt, wl.hidden, wl.inter, wl.experts, wl.top_k, host_layer, x, wr)
        dt = time.perf_counter() - t0
        rates.append(n_tokens / dt)
        secs.append(round(dt, 2))
    med = sorted(rates)[runs // 2]
    return {"value": round(med, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"median of {runs} runs of {n_tokens} decode tokens each of the MiMo-shaped "
                      f"MXFP4 layer (fp32 router, top-8, 8 experts in float64 each); run times "
                      f"{secs} s",
            "runs_tokens_per_s": [round(v, 3) for v in rates]}


def host_info():
    """CPU model and core counts from /proc/cpuinfo (physical cores = distinct
    (physical id, core id) pairs)."""
    model, cores, logical = None, set(), 0
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "processor":
                    logical += 1
                elif k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return {"cpu_model": model or platform.processor() or platform.machine(),
            "cpu_physical_cores": len(cores) or None, "cpu_logical_cpus": logical or os.cpu_count(),
            "cpu_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
            else None}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--layers", type=int, default=8, help="device copies of the layer cycled")
    ap.add_argument("--clock-warmup", type=float, default=0.3,
                    help="seconds of untimed decode steps before the warm-up steps of the "
                         "headline workload (the GPU clock ramps up under load)")
    ap.add_argument("--cpu-tokens", type=int, default=12, help="oracle tokens per run")
    ap.add_argument("--cpu-runs", type=int, default=5, help="oracle runs (median)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="decode only")
    ap.add_argument("--only", choices=["decode", "verify", "prefill", "vq_prefill", "vq_decode",
                                       "vq13_decode", "vq_verify", "copy"],
                    default=None,
                    help="run one workload without the report (for profilers)")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--replay", type=int, default=0,
                    help="with --only: also time each stage alone over this many launches")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_moe_gemv_amd as bq
    import workloads as W

    bq.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.only == "copy":
        # a plain device copy of known size (1 GiB read + 1 GiB written per
        # launch): the reference that scales HBM byte counters
        n = 1 << 30
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        c = torch.empty_like(a)
        for _ in range(args.steps):
            c.copy_(a)
        torch.cuda.synchronize()
        log(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}))
        return
    b = Bench(args, torch, bq, W)

    if args.only:
        wl = {"decode": W.DECODE, "verify": W.VERIFY, "prefill": W.PREFILL,
              "vq_prefill": W.VQ_PREFILL,
              "vq_decode": W.VQ_PREFILL.replace(tokens=1, name="mimo_vq_decode_t1"),
              "vq13_decode": W.VQ13_DECODE,
              "vq_verify": W.VERIFY.replace(fmt=W.FMT_VQ13R8, name="mimo_vq_verify_t16_skewed"),
              }[args.only]
        layers = (b.vq_layers() if wl.fmt == W_FMT_VQ else
                  b.vq13_layers() if wl.fmt == W_FMT_VQ13 else None)
        res = b.run(wl, args.steps, args.warmup, wl.tokens, profile=False, layers=layers,
                    replay=args.replay)
        log(json.dumps(res))
        return

    log("decode T=1")
    dec = b.run(W.DECODE, args.steps, args.warmup, 1, replay=args.steps,
                clock_warmup_s=args.clock_warmup)
    wl = W.DECODE
    alg = algorithmic(wl, dec["distinct_experts_last_step"], 1)
    gu_us = dec["replay_us"]["gateup"]
    achieved = alg["gateup_bytes"] / (gu_us * 1e-6) / 1e9
    roof = {"kernel": "decode_gateup_mxfp4", "bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": _traffic("decode_gateup_mxfp4", ("decode.hip", "moe_internal.h"), 1),
            "algorithmic_bytes_per_launch": alg["gateup_bytes"], "avg_launch_us": gu_us}
    step_gbs = alg["step_bytes"] / (dec["ms_per_step"] * 1e-3) / 1e9
    log("decode T=1 replayed from a captured graph")
    dec["graph_us_per_step"] = b.graph_steps(W.DECODE)
    extra = {"decode_t1": {**dec, "step_algorithmic_bytes": alg["step_bytes"],
                           "step_hbm_gbs": round(step_gbs, 1),
                           "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
                           "down_hbm_gbs": round(alg["down_bytes"] / (dec["replay_us"]["down"] * 1e-6) / 1e9, 1)}}

    if not args.no_extra:
        log("verify T=16 (skewed routing)")
        ver = b.run(W.VERIFY, max(200, args.steps // 4), 50, 16, replay=50)
        a = algorithmic(W.VERIFY, ver["distinct_experts_last_step"], 16)
        extra["verify_t16"] = {**ver, "step_algorithmic_bytes": a["step_bytes"],
                               "step_hbm_gbs": round(a["step_bytes"] / (ver["ms_per_step"] * 1e-3) / 1e9, 1)}
        log("prefill T=2048")
        pre = b.run(W.PREFILL, 30, 5, 2048, replay=10)
        extra["prefill_t2048"] = prefill_report(pre, algorithmic(W.PREFILL, W.PREFILL.experts, 2048))
        log("VQ13R8 decode T=1")
        vqd = b.run(W.VQ_PREFILL.replace(tokens=1, name="mimo_vq_decode_t1"), 1000, 200, 1,
                    layers=b.vq_layers(), replay=500)
        extra["vq_decode_t1"] = vqd
        log("VQ13R8 verify T=16 (skewed routing)")
        vqv = b.run(W.VERIFY.replace(fmt=W.FMT_VQ13R8, name="mimo_vq_verify_t16_skewed"), 100, 10,
                    16, layers=b.vq_layers(), replay=20)
        extra["vq_verify_t16"] = vqv
        log("verify-width sweep")
        sweep = {}
        for t in (1, 3, 4, 8, 16):
            wv = W.VERIFY.replace(tokens=t, name=f"mimo_verify_t{t}_skewed")
            row = {}
            for name, pth in (("decode", bq.MOE_PATH_DECODE), ("grouped", bq.MOE_PATH_PREFILL)):
                r = b.run(wv, 100, 10, t, profile=False, path=pth)
                row[name + "_us"] = round(r["ms_per_step"] * 1e3, 2)
            vq = b.run(W.VERIFY.replace(tokens=t, fmt=W.FMT_VQ13R8), 50, 5, t, profile=False,
                       layers=b.vq_layers())
            row["vq13r8_auto_us"] = round(vq["ms_per_step"] * 1e3, 2)
            row["distinct_experts"] = vq["distinct_experts_last_step"]
            sweep[f"t{t}"] = row
        extra["verify_width_sweep"] = sweep
        log("VQ13 decode T=1")
        extra["vq13_decode_t1"] = b.run(W.VQ13_DECODE, 1000, 200, 1, layers=b.vq13_layers(),
                                        replay=500)
        log("VQ13R8 prefill T=2048")
        vq = b.run(W.VQ_PREFILL, 30, 5, 2048, layers=b.vq_layers(), replay=10)
        extra["vq_prefill_t2048"] = prefill_report(
            vq, algorithmic(W.VQ_PREFILL, W.VQ_PREFILL.experts, 2048))
    if not args.no_peaks:
        extra["measured_peaks"] = measured_peaks(torch, bq, alg["step_bytes"])
        rp = extra["measured_peaks"]["read_probe_gbs_decode_step"]
        roof["frac_of_read_probe"] = round(achieved / rp, 4)
        extra["decode_t1"]["step_frac_of_read_probe"] = round(step_gbs / rp, 4)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle, {args.cpu_runs} runs of {args.cpu_tokens} decode tokens")
        cpu = cpu_baseline(b.host_layer, W, args.cpu_tokens, args.cpu_runs)

    line = {
        "metric": METRIC,
        "value": round(dec["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded MXFP4 codes/E8M0 scales, bf16 N(0,1) tokens, fp32 N(0,0.02) router)",
        "config": {"workload": wl.name, "hidden": wl.hidden, "inter": wl.inter,
                   "experts": wl.experts, "top_k": wl.top_k, "format": "mxfp4",
                   "tokens_per_step": 1, "layer_copies": args.layers},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
        "host": {**host_info(), "gpu": torch.cuda.get_device_name(0)},
        "inputs_sha256": b.input_hashes,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
