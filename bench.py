#!/usr/bin/env python
"""GDN layer throughput on one MI355X.

One step = one pass of the whole GDN hot path on Qwen3-Next-shaped synthetic inputs
(H_qk = 16, H_v = 32, d_k = d_v = 128, bf16 inputs, fp32 state pool):
  prefill : gdn_extend_gated over 8 sequences x 4096 tokens (packed varlen, zero
            initial states, final states into 8 slots of a 16-slot pool)
  decode  : gdn_decode_gated for 256 sequences x 1 token, in place on a
            [1024, 32, 128, 128] fp32 pool (256 slots touched)
Both calls take the raw gate inputs a, b (with A_log, dt_bias) and compute the decay
and write strength inside the layer kernel (the gdn_gate arithmetic, folded in).
value = (32768 + 256) tokens / step time, inputs resident in HBM.

Prints ONE JSON line.  `roofline` covers the kernel with the largest share of the
step (per-launch time from HIP events recorded on the launch stream, which is
torch's current stream); its `traffic` comes from the committed hardware-counter
summary under profiles/ when that summary was taken on the same kernel source.
`cpu_baseline` times the CPU oracle on a bounded sample of the prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --summarize-prof KT_DIR FETCH_DIR WRITE_DIR   (writes profiles/)
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN layer tokens/s (extend, decode) on 1 MI355X; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

# algorithmic work per token at the Qwen3-Next shape (H_qk=16, H_v=32, d=128)
H_QK, H_V, D = 16, 32, 128
IO_BYTES_PER_TOKEN = 2 * H_QK * D * 2 + H_V * D * 2 + H_V * D * 2 + H_V * 4   # q,k + v + out + a,b (bf16)
STATE_BYTES = H_V * D * D * 4                                                   # one slot, all heads
CHUNK = 64
EXTEND_FLOP_PER_TOKEN = H_QK * 4 * CHUNK * D + H_V * 2 * (CHUNK * D + 2 * CHUNK * D + 3 * D * D)

PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "gdn_step_prefill_8x4096_decode_256_traffic.txt")
KERNEL_SOURCES = {"extend": "hybrid_model_linear_amd/csrc/chunk.hip",
                  "decode": "hybrid_model_linear_amd/csrc/recurrent.hip",
                  "conv_prefill": "hybrid_model_linear_amd/csrc/conv.hip"}
KERNEL_NAMES = {"extend": "chunk_kernel<128, 128, false, unsigned short",
                "decode": "recurrent_kernel<128, 128, unsigned short",
                "conv_prefill": "conv_out_kernel<4, true>"}
PROF_CMD = "python bench.py --steps 20 --warmup 1000 --no-cpu-baseline --calibrate-copy-mib 1024"
PMC_CMD = "python bench.py --steps 5 --warmup 2 --no-cpu-baseline --calibrate-copy-mib 1024"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # ~0.6 s of warm-up: the GPU's clocks settle before the timed region
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (for counter scaling)")
    ap.add_argument("--summarize-prof", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="summarize rocprofv3 outputs of this script into profiles/ and exit")
    return ap.parse_args()


def source_sha(kind):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kind]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# ------------------------------------------------------------------ counter summaries
def _csv_rows(d, pattern):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_prof(kt_dir, fetch_dir, write_dir):
    """profiles/ text summaries of three rocprofv3 runs of PROF_CMD: the kernel-trace
    statistics, and FETCH_SIZE / WRITE_SIZE per dispatch scaled by what the same
    counters read for the 1 GiB copy kernel (torch.mul: reads and writes 1 GiB)."""
    os.makedirs(PROFILES, exist_ok=True)
    stats = _csv_rows(kt_dir, "*kernel_stats.csv")
    lines = ["# rocprofv3 kernel-trace statistics of the bench command",
             f"# command (repository root): export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             f"-d <dir> -o bench -- {PROF_CMD}",
             f"# summarized by: python bench.py --summarize-prof <kt_dir> <fetch_dir> <write_dir>",
             f"# kernel sources: chunk.hip sha256 {source_sha('extend')}, recurrent.hip sha256 {source_sha('decode')}, "
             f"conv.hip sha256 {source_sha('conv_prefill')}",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in stats:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}  {r['Name'][:110]}")
    with open(os.path.join(PROFILES, "gdn_step_prefill_8x4096_decode_256_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(d, counter):
        vals = {}
        for r in _csv_rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def pick(vals, needle):
        for k, v in vals.items():
            if needle in k:
                return sum(v) / len(v), len(v)
        raise SystemExit(f"kernel {needle!r} not found")
    copy_kib = 1024 * 1024.0                       # 1 GiB read and written by the copy

    def pick_copy(vals):                           # the largest MulFunctor dispatch
        return max(max(v) for k, v in vals.items() if "MulFunctor" in k)
    cf, cw = pick_copy(fetch), pick_copy(write)
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    out = ["# HBM traffic per dispatch from rocprofv3 counters (KiB), scaled by the copy calibration",
           f"# command (fetch, repository root): export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- {PMC_CMD}",
           f"# command (write, repository root): export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o bench -- {PMC_CMD}",
           "# summarized by: python bench.py --summarize-prof <kt_dir> <fetch_dir> <write_dir>",
           f"copy_fetch_kib {cf:.1f}", f"copy_write_kib {cw:.1f}",
           f"fetch_scale {f_scale:.4f}", f"write_scale {w_scale:.4f}"]
    for kind in ("extend", "decode", "conv_prefill"):
        if kind == "conv_prefill" and not any(KERNEL_NAMES[kind] in k for k in fetch):
            continue                                # a profile without the conv leg
        fk, n = pick(fetch, KERNEL_NAMES[kind])
        wk, _ = pick(write, KERNEL_NAMES[kind])
        out += [f"{kind}_source_sha256 {source_sha(kind)}", f"{kind}_dispatches {n}",
                f"{kind}_fetch_kib {fk:.1f}", f"{kind}_write_kib {wk:.1f}",
                f"{kind}_traffic_bytes {int(round((fk * f_scale + wk * w_scale) * 1024))}"]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(lines + out))


def measured_traffic(kind):
    """Scaled counter traffic per launch of `kind`, or None when no summary exists or
    it was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(None, 1) for l in f.read().splitlines() if l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get(f"{kind}_source_sha256", "").strip() != source_sha(kind):
        return None
    return int(kv[f"{kind}_traffic_bytes"])


# ------------------------------------------------------------------ CPU oracle baseline
def cpu_baseline(ext, seconds):
    """The float64 oracle, token by token over all 32 heads, on the prefill workload's
    sequences in order (64-token blocks carrying the state), as many tokens as fit in
    `seconds` of CPU time on one thread; tokens/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    ctx = threadpool_limits(1) if threadpool_limits else None
    blk = 64
    nq = H_QK * D
    cu = ext.cu_seqlens
    done, spent, seqs = 0, 0.0, 0
    try:
        for s in range(len(cu) - 1):
            t0, t1 = int(cu[s]), int(cu[s + 1])
            S = np.zeros((1, H_V, D, D))
            seqs += 1
            for b0 in range(t0, t1, blk):
                if spent >= seconds:
                    break
                b1 = min(t1, b0 + blk)
                n = b1 - b0
                mixed = ext.mixed_qkv[b0:b1].float().cpu().numpy()
                a = ext.a[b0:b1].float().cpu().numpy()
                b = ext.b[b0:b1].float().cpu().numpy()
                q = mixed[:, :nq].reshape(n, H_QK, D)
                k = mixed[:, nq:2 * nq].reshape(n, H_QK, D)
                v = mixed[:, 2 * nq:].reshape(n, H_V, D)
                t = time.perf_counter()
                _, _, fin = oracle.gdn_extend(q, k, v, a, b, ext.A_log, ext.dt_bias,
                                              np.array([0, n]), np.array([0]), np.array([int(b0 > t0)]),
                                              S, ext.scale)
                spent += time.perf_counter() - t
                S = fin[0][None]
                done += n
            if spent >= seconds:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": round(done / spent, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 oracle, first {done} tokens of the prefill workload ({seqs} sequence(s) "
                      f"of 4096, state carried in 64-token blocks) x all {H_V} heads, {spent:.1f} s on one thread"}


def bench_conv(torch, gdn, T_e, n_seq, T_d, steps):
    """The short causal conv in front of the layer (width 4, silu, bf16 conv states),
    timed on its own: it is not part of the step.  Prefill: the step's 8 x 4096 tokens
    of the q | k | v width (8192 channels) from earlier states; decode: 256 rows on a
    1024-slot conv pool.  HIP events on torch's current stream, the launch stream."""
    dev, K, Dc = "cuda", 4, 2 * H_QK * D + H_V * D
    g = torch.Generator(device=dev).manual_seed(5)
    bf = lambda *shape: torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    w, b = bf(Dc, K) * 0.5, bf(Dc) * 0.5
    L = T_e // n_seq
    cu = torch.arange(0, T_e + 1, L, dtype=torch.int32, device=dev)
    x_e, out_e, pool_e = bf(T_e, Dc), torch.empty((T_e, Dc), dtype=torch.bfloat16, device=dev), bf(16, Dc, K - 1)
    slot_e = torch.arange(n_seq, dtype=torch.int32, device=dev)
    x_d, out_d, pool_d = bf(T_d, Dc), torch.empty((T_d, Dc), dtype=torch.bfloat16, device=dev), bf(1024, Dc, K - 1)
    slot_d = torch.randperm(1024, generator=g, device=dev)[:T_d].to(torch.int32)
    calls = {"prefill": lambda: gdn.conv1d(x_e, w, b, cu, slot_e, pool_e, out=out_e),
             "decode": lambda: gdn.conv1d_update(x_d, w, b, slot_d, pool_d, out=out_d)}
    state = Dc * (K - 1) * 2
    work = {"prefill": T_e * Dc * 4 + n_seq * 2 * state, "decode": T_d * (Dc * 4 + 2 * state)}
    res = {"workload": f"prefill {n_seq}x{L} and decode {T_d}x1, {Dc} channels, width {K}"}
    for name, fn in calls.items():
        for _ in range(20):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        gbs = work[name] / (us * 1e-6) / 1e9
        res[name] = {"avg_us": round(us, 2), "bytes": work[name], "GB_s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    # counter traffic of the output pass (the state pass moves 0.4 MB)
    res["prefill"]["traffic_bytes_output_pass"] = measured_traffic("conv_prefill")
    return res


def main():
    args = parse()
    if args.summarize_prof:
        summarize_prof(*args.summarize_prof)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer needs no collective; heads and "
              f"sequences shard independently); --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import hybrid_model_linear_amd as gdn
    from hybrid_model_linear_amd import synth

    gdn.load()
    dev = "cuda"
    torch.cuda.set_device(0)
    # ---------------- inputs (resident in HBM before timing)
    ext = synth.device_config2_prefill()
    dec = synth.device_config1_decode()
    pool_e = synth.device_pool(ext)
    pool_d = synth.device_pool(dec)

    def prep(case):
        q, k, v = gdn.split_mixed_qkv(case.mixed_qkv, case.H_qk, case.H_v, case.d_k, case.d_v)
        t = lambda x, dt: torch.from_numpy(x).to(dev, dt)
        return dict(q=q, k=k, v=v, a=case.a, b=case.b, A_log=t(case.A_log, torch.float32),
                    dt_bias=t(case.dt_bias, torch.float32), cu=t(case.cu_seqlens, torch.int32),
                    slot=t(case.slot, torch.int32), has_init=t(case.has_init, torch.int32),
                    out=torch.empty((case.T, case.H_v, case.d_v), dtype=torch.bfloat16, device=dev))
    E, Dd = prep(ext), prep(dec)
    T_e, T_d = ext.T, dec.T
    maxlen = int(max(ext.cu_seqlens[1:] - ext.cu_seqlens[:-1]))

    if args.calibrate_copy_mib:
        # a plain streaming kernel of known traffic (reads and writes N bytes) whose
        # FETCH_SIZE / WRITE_SIZE readings scale the counters of the GDN kernels
        src = torch.ones((args.calibrate_copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    names = ["extend", "decode"]
    gate_e = gdn.gdn_gate_inputs(E["a"], E["b"], E["A_log"], E["dt_bias"])
    gate_d = gdn.gdn_gate_inputs(Dd["a"], Dd["b"], Dd["A_log"], Dd["dt_bias"])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        gdn.extend(E["q"], E["k"], E["v"], None, None, E["cu"], E["slot"], pool_e,
                   has_init=E["has_init"], scale=ext.scale, out=E["out"], max_seqlen=maxlen,
                   gate=gate_e)
        mark(1)
        gdn.decode(Dd["q"], Dd["k"], Dd["v"], None, None, Dd["slot"], pool_d,
                   scale=dec.scale, out=Dd["out"], gate=gate_d)
        mark(2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(evs[s])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    per = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i, n in enumerate(names)}
    print(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    # ---------------- algorithmic work per launch
    work = {
        "extend": dict(bytes=T_e * IO_BYTES_PER_TOKEN + ext.N * STATE_BYTES,   # zero init: write only
                       flop=T_e * EXTEND_FLOP_PER_TOKEN),
        "decode": dict(bytes=T_d * (IO_BYTES_PER_TOKEN + 2 * STATE_BYTES), flop=T_d * 7 * H_V * D * D),
    }
    kernels = {}
    for n in names:
        sec = per[n] * 1e-3
        gbs = work[n]["bytes"] / sec / 1e9
        tfs = work[n]["flop"] / sec / 1e12
        kernels[n] = {"avg_us": round(per[n] * 1e3, 2), "bytes": work[n]["bytes"],
                      "flop": work[n]["flop"], "GB_s": round(gbs, 1), "TFLOP_s": round(tfs, 2),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)}
    for n in ("extend", "decode"):
        kernels[n]["traffic_bytes"] = measured_traffic(n)
    dom = max(("extend", "decode"), key=lambda n: per[n])
    kd = kernels[dom]
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    ai = work[dom]["flop"] / work[dom]["bytes"]
    roofline = {"kernel": dom, "bound": "hbm" if ai < ridge else "mfma",
                "achieved": kd["GB_s"] if ai < ridge else kd["TFLOP_s"],
                "peak": HBM_PEAK_GBS if ai < ridge else MFMA_BF16_PEAK_TFLOPS,
                "unit": "GB/s" if ai < ridge else "TFLOP/s",
                "frac": kd["hbm_frac"] if ai < ridge else kd["mfma_frac"],
                "traffic": kd["traffic_bytes"], "arith_intensity": round(ai, 1),
                "mfma_frac": kd["mfma_frac"], "avg_launch_us": kd["avg_us"]}
    tokens = T_e + T_d
    result = {
        "metric": METRIC, "value": round(tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GDN layer step: extend 8x4096 (zero init) + decode 256x1 "
                               "(pool [1024,32,128,128] fp32)",
                   "H_qk": H_QK, "H_v": H_V, "d_k": D, "d_v": D, "chunk": CHUNK,
                   "extend_tokens": T_e, "decode_tokens": T_d, "state": "fp32"},
        "roofline": roofline,
        "phases": {"extend_tokens_per_s": round(T_e / (per["extend"] * 1e-3), 1),
                   "decode_tokens_per_s": round(T_d / (per["decode"] * 1e-3), 1)},
        "kernels": kernels,
    }
    result["conv1d"] = bench_conv(torch, gdn, T_e, ext.N, T_d, args.steps)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(ext, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
