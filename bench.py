"""Benchmark of the attention forward on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  * attn_fwd over the whole batch (bf16 workloads without K/V blocks),
  * attn_fwd_f32 (fp32 workload), attn_fwd_fp8 (fp8 workload),
  * n_blocks x attn_fwd_kvblock plus the merges (block-streamed workload).
W untimed warm-up steps, then K steps back to back on one stream, bracketed
by HIP events recorded on that stream (torch.cuda.Event on the stream the
kernels are launched on) and device synchronisation.  The warm-up runs at
least --warmup steps (default 10) and at least 2 s: an idle MI355X needs
about 0.1-0.2 s of load to leave its low clocks (a 5-step warm-up of the
causal B8 H16 N2048 workload, 1 ms, measures ~665 instead of ~840 TFLOP/s),
and two seconds of GPU work also make the run visible to a utilisation
sampler next to the CPU baseline's second of host work.
The JSON line's "warmup" is the requested minimum; "warmup_steps_run" and
"warmup_s" are what actually ran.  Inputs are
resident in HBM before the timed region starts.  Prints one JSON line.

The default workload is the causal bf16 B=8 H=16 N=2048 d=128 attention
(TFLOP/s = 4*B*H*N^2*d/2 / time).  The CPU baseline is the fp64 oracle timed
on a bounded sample of the same workload (whole heads, all rows).

The W4A16 workloads (--workload w4a16_...) time one w4a16_gemm call per step,
cycling through several copies of the weights so that every call reads its
weights from HBM rather than from the last-level cache; the figure is GB/s of
the bytes a call must move (packed weights, scales, zero points, activations
in, outputs out) against the 8 TB/s HBM peak.
"""
import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2, "f32": 157.3}  # dense MFMA, 256 CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E

# rocprofv3 FETCH_SIZE/WRITE_SIZE summaries (copy-calibrated) per workload; the
# figure is reported only while the kernel sources still hash to the value the
# counters were taken with.  Bytes per step: all kernel launches of one step.
TRAFFIC_PROFILES = {
    w: f"profiles/{w}_hbm_traffic.txt"
    for w in (
        "bf16_causal_B8_H16_N2048_d128",
        "bf16_causal_B1_H8_N32768_d128",
        "bf16_kvblocks_B1_H16_Nq8192_Nk65536x8_d128",
        "bf16_causal_ring_B1_H16_N65536_R8_d128",
        "fp8_B4_H16_N4096_d128",
        "fp8_norot_qk16_B4_H16_N4096_d128",
        "bwd_bf16_causal_B8_H16_N2048_d128",
        "f32_B1_H2_N256_d64",
        "w4a16_decode_M16_N28672_K8192_G128",
        "w4a16_decode_M16_N8192_K28672_G128",
    )
}


def measured_traffic(workload):
    import hashlib

    path = TRAFFIC_PROFILES.get(workload)
    if not path or not os.path.exists(os.path.join(REPO, path)):
        return None
    fields = {}
    with open(os.path.join(REPO, path)) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for src in fields["kernel sources"].split():
            with open(os.path.join(REPO, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["kernel_source_sha256"]:
            return None
        return int(fields["traffic_bytes_per_step"])
    except (KeyError, OSError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="minimum untimed warm-up steps (default 10); the warm-up also lasts at least "
                         "WARMUP_SECONDS")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-measured-peak", action="store_true",
                    help="skip the matrix-core peak loop that follows the timed region")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain copy kernel of known size (HBM counter calibration)")
    return ap.parse_args()


WARMUP_SECONDS = 2.0


def warm_up(step, warmup):
    """Run the untimed warm-up: at least `warmup` steps (10 when None) and at
    least WARMUP_SECONDS of them (the host waits for the GPU every 8 steps, so
    the time is the GPU's).  Returns (steps run, seconds)."""
    import torch

    min_steps = 10 if warmup is None else max(0, warmup)
    n, t0 = 0, time.perf_counter()
    while n < min_steps or time.perf_counter() - t0 < WARMUP_SECONDS:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


MFMA_KINDS = {"bf16": 0, "f16": 1, "fp8": 2, "f32": 3}


def mfma_peak_run(eta, kind, iters, stream, repeats=5):
    """Median TFLOP/s of `repeats` launches of the matrix-core loop (one 8-wavefront
    workgroup per compute unit), each timed with events on `stream`."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty((cus * eta.MFMA_PEAK_THREADS,), device="cuda")
    flop = eta.mfma_peak_flop(kind, cus, iters)
    eta.mfma_peak(kind, cus, iters, out, stream)  # untimed first launch
    times = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        eta.mfma_peak(kind, cus, iters, out, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    return flop / (ms * 1e-3) / 1e12, ms, cus, flop


def measured_peak(eta, dtype, stream):
    """Measured dense matrix-core peak for the workload's dtype, run right after the timed
    region (the clocks are still at their working level).  The fp8 path's Q.K runs at the fp8
    rate; its figure is reported against the fp8 loop."""
    kind = {"bf16": "bf16", "fp8": "fp8", "f32": "f32"}[dtype]
    iters = {"bf16": 20000, "fp8": 10000, "f32": 5000}[kind]
    tf, ms, cus, _ = mfma_peak_run(eta, MFMA_KINDS[kind], iters, stream)
    return {"kind": kind, "value": round(tf, 1), "unit": "TFLOP/s", "ms_per_launch": round(ms, 4),
            "workgroups": cus, "iters": iters,
            "loop": "attn_mfma_peak: 8 wavefronts per compute unit, 4 independent MFMA chains each"}


def bench_mfma(args, name, cfg):
    """The matrix-core throughput loop alone: TFLOP/s against the datasheet's dense peak."""
    import torch

    import exact_tiled_attention_15_amd as eta

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    kind = cfg["mfma"]
    iters = cfg["iters"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty((cus * eta.MFMA_PEAK_THREADS,), device="cuda")
    step = lambda: eta.mfma_peak(MFMA_KINDS[kind], cus, iters, out, stream)
    warmup, warmup_s = warm_up(step, args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    flop = eta.mfma_peak_flop(MFMA_KINDS[kind], cus, iters)
    tf = flop / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[kind]
    out_line = {
        "metric": f"dense {kind} MFMA throughput loop TFLOP/s and % of MI355X datasheet peak",
        "value": round(tf, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 10 if args.warmup is None else args.warmup,
        "warmup_steps_run": warmup,
        "warmup_s": round(warmup_s, 3),
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kind,
        "data": "register operands, no memory traffic",
        "config": {"workload": name, "workgroups": cus, "threads": eta.MFMA_PEAK_THREADS, "iters": iters,
                   "chains_per_wavefront": 4},
        "pct_of_peak": round(100 * tf / peak, 2),
        "wall_s_timed": round(t_wall, 4),
        "roofline": {"bound": "mfma", "kernel": f"mfma_peak_kernel<{MFMA_KINDS[kind]}>", "achieved": round(tf, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None,
                     "launches_per_step": 1},
        "cpu_baseline": None,
    }
    print(json.dumps(out_line), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark measures one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by (batch, head) and by ring hops, which no run here exercises.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_15_amd as eta
    from exact_tiled_attention_15_amd import configs, inputs

    name = args.workload or configs.HEADLINE
    cfg = configs.WORKLOADS[name]
    if cfg.get("kind") == "w4a16":
        return bench_w4a16(args, name, cfg)
    if cfg.get("kind") == "mfma":
        return bench_mfma(args, name, cfg)
    seed = configs.seed_of(name)
    B, H, Nq, Nk, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"]
    causal = cfg["causal"]
    scale = configs.scale_of(name)
    dtype = cfg["dtype"]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    x = inputs.make_inputs(cfg, seed, rotate=cfg.get("rotate", False))
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    if dtype == "bf16" and cfg.get("backward"):
        q, k, v = bf(x["q"]), bf(x["k"]), bf(x["v"])
        do = bf(inputs.bf16_bits(inputs.normal_f32((B, H, Nq, d), seed, 6)))
        o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")
        eta.attn_fwd(q, k, v, o, lse, causal, scale, stream)  # the forward the gradients belong to
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        work = torch.empty((eta.bwd_work_floats(B, H, Nq),), device="cuda")
        step = lambda: eta.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, work, causal, scale, stream)
        kernel = "bwd_delta_kernel + bwd_dkdv_kernel + bwd_dq_kernel"
        launches = 3
    elif dtype == "bf16" and "n_blocks" not in cfg:
        q, k, v = bf(x["q"]), bf(x["k"]), bf(x["v"])
        o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")
        step = lambda: eta.attn_fwd(q, k, v, o, lse, causal, scale, stream)
        kernel = "fwd_bf16_kernel"
        launches = 1
    elif dtype == "bf16" and cfg.get("host_kv"):
        nb = cfg["n_blocks"]
        blk = Nk // nb
        q = bf(x["q"])
        # blocks in page-locked host memory, hop order = block order
        kh = [torch.from_numpy(np.ascontiguousarray(x["k"][:, :, i * blk:(i + 1) * blk]).view(np.int16))
              .view(torch.bfloat16).pin_memory() for i in range(nb)]
        vh = [torch.from_numpy(np.ascontiguousarray(x["v"][:, :, i * blk:(i + 1) * blk]).view(np.int16))
              .view(torch.bfloat16).pin_memory() for i in range(nb)]
        pos = [i * blk for i in range(nb)]
        o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")
        work = torch.empty((eta.ring_work_floats(B, H, Nq, d),), device="cuda")
        stage = torch.empty((eta.ring_stage_bytes(B, H, blk, d),), dtype=torch.uint8, device="cuda")
        step = lambda: eta.attn_fwd_ring_host(q, kh, vh, pos, o, lse, work, stage, causal, 0, scale, stream)
        kernel = "fwd_bf16_kernel (state epilogue) + merge_kernel, via attn_fwd_ring_host"
        launches = 2 * nb - 1
        transfer = host_kv_parts(args, eta, q, kh, vh, pos, o, lse, work, causal, scale, stream)
    elif dtype == "bf16" and cfg.get("ring"):
        nb = cfg["n_blocks"]
        blk = Nk // nb
        q, k, v = bf(x["q"]), bf(x["k"]), bf(x["v"])
        kbs = [k[:, :, i * blk:(i + 1) * blk].contiguous() for i in range(nb)]
        vbs = [v[:, :, i * blk:(i + 1) * blk].contiguous() for i in range(nb)]
        del k, v
        hops = configs.ring_hops(name)
        kh, vh, pos = [kbs[b] for b, _ in hops], [vbs[b] for b, _ in hops], [kp for _, kp in hops]
        o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")
        work = torch.empty((eta.ring_work_floats(B, H, Nq, d),), device="cuda")
        step = lambda: eta.attn_fwd_ring(q, kh, vh, pos, o, lse, work, causal, cfg["q_pos0"], scale, stream)
        kernel = "fwd_bf16_kernel (state epilogue) + merge_kernel, via attn_fwd_ring"
        launches = 2 * nb - 1
    elif dtype == "bf16":
        nb = cfg["n_blocks"]
        blk = Nk // nb
        q, k, v = bf(x["q"]), bf(x["k"]), bf(x["v"])
        kbs = [k[:, :, i * blk:(i + 1) * blk].contiguous() for i in range(nb)]
        vbs = [v[:, :, i * blk:(i + 1) * blk].contiguous() for i in range(nb)]
        del k, v
        acc = [torch.empty((B, H, Nq, d), device="cuda"), torch.empty((B, H, Nq), device="cuda"),
               torch.empty((B, H, Nq), device="cuda")]
        part = [torch.empty_like(t) for t in acc]
        o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")

        def step():
            eta.attn_fwd_kvblock(q, kbs[0], vbs[0], *acc, False, 0, 0, scale, stream)
            for i in range(1, nb):
                eta.attn_fwd_kvblock(q, kbs[i], vbs[i], *part, False, 0, i * blk, scale, stream)
                last = i == nb - 1
                eta.attn_merge(*acc, *part, o if last else None, lse if last else None, stream)
        kernel = "fwd_bf16_kernel (state epilogue) + merge_kernel"
        launches = nb
    elif dtype == "f32":
        q, k, v = dv(x["q"]), dv(x["k"]), dv(x["v"])
        o = torch.empty((B, H, Nq, d), device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")
        step = lambda: eta.attn_fwd_f32(q, k, v, o, lse, causal, scale, stream)
        kernel = "fwd_f32_kernel"
        launches = 1
    else:
        t = {n: dv(x[n]) for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale")}
        o = torch.empty((B, H, Nq, d), device="cuda")
        lse = torch.empty((B, H, Nq), device="cuda")
        if cfg.get("pv4"):
            direct = bool(cfg.get("direct_p"))
            step = lambda: eta.attn_fwd_fp8_pv4(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"],
                                                t["v_scale"], o, lse, causal, scale, direct, stream)
        else:
            fp8_fn = (eta.attn_fwd_fp8_pv8 if cfg.get("pv8") else
                      eta.attn_fwd_fp8_qk16 if cfg.get("qk16") else eta.attn_fwd_fp8)
            step = lambda: fp8_fn(t["q8"], t["k8"], t["v8"], t["q_scale"], t["k_scale"], t["v_scale"],
                                  o, lse, causal, scale, stream)
        kernel = "fwd_fp8_kernel"
        launches = 1

    if not cfg.get("host_kv"):
        transfer = None
    flop = configs.workload_flops(name)
    warmup, warmup_s = warm_up(step, args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    tflops = flop / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]

    if args.copy_calibration:
        # plain copy of a known size: 256 MiB read + 256 MiB written
        src = torch.ones(64 << 20, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()

    mpeak = None if args.no_measured_peak else measured_peak(eta, dtype, stream)
    if mpeak is not None:
        mpeak["frac"] = round(tflops / mpeak["value"], 4)
    roofline = {
        "bound": "mfma",
        "kernel": kernel,
        "achieved": round(tflops, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(tflops / peak, 4),
        "traffic": measured_traffic(name),
        "traffic_unit": "bytes per step, all launches (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "launches_per_step": launches,
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(name, cfg, seed, x, args.cpu_seconds)

    out = {
        "metric": ("attention bwd TFLOP/s (bf16 d=128, causal; FLOPs = 2.5x the forward's) and % of MI355X "
                   "dense MFMA peak" if cfg.get("backward") else
                   "attention fwd TFLOP/s (bf16 d=128, causal) and % of MI355X dense MFMA peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 10 if args.warmup is None else args.warmup,
        "warmup_steps_run": warmup,
        "warmup_s": round(warmup_s, 3),
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": name, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "causal": causal,
                   "scale": scale, "seed": seed},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "pct_of_measured_peak": None if mpeak is None else round(100 * mpeak["frac"], 2),
        "wall_s_timed": round(t_wall, 4),
        "roofline": roofline,
        "measured_peak": mpeak,
        "cpu_baseline": cpu,
    }
    if transfer is not None:
        transfer["total_ms"] = round(ms, 4)
        c, g = transfer["copy_ms"], transfer["compute_ms"]
        # share of the shorter of the two parts that ran under the other
        transfer["hidden_frac"] = round(max(0.0, c + g - ms) / min(c, g), 4)
        out["transfer"] = transfer
        out["data"] += "; K/V blocks in page-locked host memory, copied to the GPU inside the timed step"
    print(json.dumps(out), flush=True)


def cpu_baseline(name, cfg, seed, x, target_s):
    """The fp64 oracle on whole heads of the same workload, sized to ~target_s."""
    import oracle
    from exact_tiled_attention_15_amd import configs

    B, H, Nq, Nk, d, causal = cfg["B"], cfg["H"], cfg["Nq"], cfg["Nk"], cfg["d"], cfg["causal"]
    scale = configs.scale_of(name)
    dtype = cfg["dtype"]

    def head(b, h):
        if dtype == "bf16":
            dec = lambda a: oracle.decode_bf16(a[b:b + 1, h:h + 1])
            return dec(x["q"]), dec(x["k"]), dec(x["v"])
        if dtype == "f32":
            return tuple(x[n][b:b + 1, h:h + 1].astype(np.float64) for n in ("q", "k", "v"))
        dq = lambda c, s: oracle.decode_e4m3(c[b:b + 1, h:h + 1], s[b:b + 1, h:h + 1])
        return dq(x["q8"], x["q_scale"]), dq(x["k8"], x["k_scale"]), dq(x["v8"], x["v_scale"])

    # Size the sample with one probe of 32 rows, then run whole heads.
    q, k, v = head(0, 0)
    probe_rows = np.arange(Nq - 32, Nq, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, causal, scale, rows=probe_rows)
    t_probe = time.perf_counter() - t0
    keys_probe = float(sum((i + Nk - Nq + 1) if causal else Nk for i in probe_rows))
    keys_head = float(sum((i + Nk - Nq + 1) if causal else Nk for i in range(Nq)))
    t_head = max(t_probe * keys_head / keys_probe, 1e-6)
    backward = bool(cfg.get("backward"))
    if backward:  # the gradient costs about four forward passes in the oracle
        t_head *= 4.0
        from exact_tiled_attention_15_amd import inputs
        dob = inputs.bf16_bits(inputs.normal_f32((B, H, Nq, d), seed, 6))
    n_heads = int(max(1, min(B * H, target_s / t_head)))
    flop = 0.0
    elapsed = 0.0  # oracle time only; decoding the slice's inputs is not counted
    for u in range(n_heads):
        b, h = divmod(u, H)
        q, k, v = head(b, h)
        if backward:
            do = oracle.decode_bf16(dob[b:b + 1, h:h + 1])
            tt = time.perf_counter()
            oracle.attention_bwd(q, k, v, do, causal, scale)
            elapsed += time.perf_counter() - tt
            flop += 2.5 * 4.0 * d * keys_head
            continue
        tt = time.perf_counter()
        oracle.attention(q, k, v, causal, scale)
        elapsed += time.perf_counter() - tt
        flop += 4.0 * d * keys_head
    return {
        "value": round(flop / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n_heads} of {B * H} (b,h) slices, all {Nq} rows x {'causal' if causal else 'all'} keys"
                  f"{', gradients dq/dk/dv' if backward else ''}, "
                  f"fp64, {elapsed:.1f} s on {cpu_model()}",
        "flop": flop,
        "seconds": round(elapsed, 3),
    }


def host_kv_parts(args, eta, q, kh, vh, pos, o, lse, work, causal, scale, stream):
    """The two parts of a host-streamed ring step timed alone: the host-to-device copies of
    every block (into two device slots, as the step does) and the attention over the same
    blocks already resident on the device (attn_fwd_ring)."""
    import torch

    kd = [t.cuda() for t in kh]
    vd = [t.cuda() for t in vh]
    slots = [torch.empty_like(kd[0]) for _ in range(4)]

    def copies():
        for i in range(len(kh)):
            slots[2 * (i & 1)].copy_(kh[i], non_blocking=True)
            slots[2 * (i & 1) + 1].copy_(vh[i], non_blocking=True)

    def compute():
        eta.attn_fwd_ring(q, kd, vd, pos, o, lse, work, causal, 0, scale, stream)

    def timed(fn, n):
        warm_up(fn, args.warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(3, args.steps // 2)
    copy_ms = timed(copies, n)
    compute_ms = timed(compute, n)
    nbytes = 2 * sum(t.numel() * t.element_size() for t in kh)
    del kd, vd, slots
    torch.cuda.empty_cache()
    return {"bytes_per_step": nbytes, "copy_ms": round(copy_ms, 4), "copy_GBps": round(nbytes / copy_ms / 1e6, 2),
            "compute_ms": round(compute_ms, 4)}


def bench_w4a16(args, name, cfg):
    import torch

    import exact_tiled_attention_15_amd as eta
    from exact_tiled_attention_15_amd import configs, inputs

    M, N, K, G = cfg["M"], cfg["N"], cfg["K"], cfg["group"]
    copies = cfg["weight_copies"]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    host = [inputs.make_w4a16_inputs(M, N, K, G, cfg["seed"] + 100 * c) for c in range(copies)]
    x = torch.from_numpy(host[0]["x"].view(np.int16)).view(torch.float16).cuda()
    ws = []
    for h in host:
        ws.append((torch.from_numpy(h["packed"].view(np.int32)).cuda(),
                   torch.from_numpy(h["scales"].view(np.int16)).view(torch.float16).cuda(),
                   torch.from_numpy(h["zeros"]).cuda()))
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    nw = eta.w4a16_work_floats(M, N, K)
    work = torch.empty((nw,), device="cuda") if nw else None
    state = {"i": 0}

    def step():
        p, sc, z = ws[state["i"] % copies]
        state["i"] += 1
        eta.w4a16_gemm(x, p, sc, z, y, work, G, stream)

    warmup, warmup_s = warm_up(step, args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    if args.copy_calibration:
        # plain copy of a known size: 256 MiB read + 256 MiB written
        src = torch.ones(64 << 20, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
    nbytes = configs.w4a16_bytes(name)
    gbs = nbytes / (ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": "w4a16_kernel" + (" + w4a16_reduce_kernel" if nw else ""),
        "achieved": round(gbs, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(gbs / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(name),
        "traffic_unit": "bytes per step, all launches (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "algorithmic_bytes": nbytes,
        "launches_per_step": 2 if nw else 1,
    }
    cpu = None if args.no_cpu_baseline else cpu_baseline_w4a16(cfg, host[0], args.cpu_seconds)
    out = {
        "metric": "W4A16 decode linear layer GB/s (packed 4-bit weights + group scales/zero points + fp16 "
                  "activations and outputs) and % of MI355X HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 10 if args.warmup is None else args.warmup,
        "warmup_steps_run": warmup,
        "warmup_s": round(warmup_s, 3),
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": f"synthetic (seeded random 4-bit codes, scales and zero points; N(0,1) activations; "
                f"{copies} weight copies in rotation)",
        "config": {"workload": name, "M": M, "N": N, "K": K, "group": G, "seed": cfg["seed"]},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "wall_s_timed": round(t_wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_w4a16(cfg, h, target_s):
    """The fp64 oracle on a subset of weight rows (all tokens, all of K), sized to ~target_s."""
    import oracle
    from exact_tiled_attention_15_amd import inputs

    M, N, K, G = cfg["M"], cfg["N"], cfg["K"], cfg["group"]
    probe = inputs.row_subset(N, 64, seed=12)
    t0 = time.perf_counter()
    oracle.w4a16(h["x"], h["packed"][probe], h["zeros"][probe], h["scales"][probe], G)
    t_probe = max(time.perf_counter() - t0, 1e-6)
    R = int(max(64, min(N, 64 * target_s / t_probe)))
    rows = inputs.row_subset(N, R, seed=13)
    p, z, sc = h["packed"][rows], h["zeros"][rows], h["scales"][rows]
    t0 = time.perf_counter()
    oracle.w4a16(h["x"], p, z, sc, G)
    elapsed = time.perf_counter() - t0
    nbytes = R * (K // 2 + (K // G) * 3) + M * K * 2 + M * R * 2
    return {
        "value": round(nbytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{R} of {N} weight rows, all {M} tokens x {K} inputs, fp64, {elapsed:.1f} s on {cpu_model()}",
        "bytes": nbytes,
        "seconds": round(elapsed, 3),
    }


if __name__ == "__main__":
    main()
