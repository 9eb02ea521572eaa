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
`measured_peaks` holds the box's own copy bandwidth and bf16 MFMA rate (the library's
probes), and every kernel entry its fraction of them beside the published peaks.
`cpu_baseline` times the float64 CPU oracle on the whole prefill workload over the
host's cores (one single-threaded worker process per unit; the one-thread rate beside
it).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--no-cpu-baseline]

Before the W warm-up steps the step runs back to back for --settle-ms (default 250
ms, untimed): the GPU's clocks ramp up over the first ~50 ms of sustained load.
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
                  "ssd": "hybrid_model_linear_amd/csrc/ssd.hip",
                  "decode": "hybrid_model_linear_amd/csrc/recurrent.hip",
                  "conv_prefill": "hybrid_model_linear_amd/csrc/conv.hip"}
KERNEL_NAMES = {"extend": "chunk_kernel<128, 128, false, unsigned short",
                "decode": "recurrent_kernel<128, 128, unsigned short",
                "conv_prefill": "conv_out_kernel<4, true>"}
PROF_CMD = "python bench.py --steps 20 --warmup 20 --no-cpu-baseline --no-configs --calibrate-copy-mib 1024"
PMC_CMD = "python bench.py --steps 5 --warmup 2 --settle-ms 0 --no-cpu-baseline --no-configs --calibrate-copy-mib 1024"
SQ_PASSES = (("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_MFMA",
              "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS"),
             ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_INSTS_SALU",
              "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_VALU_MFMA_COEXEC_CYCLES",
              "SQ_WAIT_ANY"))
SQ_FILE = os.path.join(PROFILES, "gdn_step_prefill_8x4096_decode_256_sq_counters.txt")
CONFIGS_PROF_CMD = "python bench.py --steps 20 --no-cpu-baseline --configs-only"
CONFIGS_STATS_FILE = os.path.join(PROFILES, "gdn_ragged_verify_ssd128_kernel_stats.txt")
SSD_PMC_CMD = "python bench.py --steps 5 --no-cpu-baseline --configs-only --ssd-only --calibrate-copy-mib 1024"
SSD_COUNTERS_FILE = os.path.join(PROFILES, "gdn_ssd_chunk128_2x8192x80_counters.txt")
SSD_KERNELS = (("prep", "ssd_prep_kernel"), ("state_pass", "ssd_kernel<unsigned short, true, false"),
               ("full_pass", "ssd_kernel<unsigned short, true, true"))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # The GPU's clocks ramp up over the first ~50 ms of sustained load (the extend
    # kernel's time falls from ~360 to ~265 us per call): before the warm-up steps, the
    # step runs back to back for this long, untimed, so that the timed steps see the
    # sustained clock that a serving loop runs at.
    ap.add_argument("--settle-ms", type=float, default=250.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the ragged, verify and delta-off workloads")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (for counter scaling)")
    ap.add_argument("--configs-only", action="store_true",
                    help="time only the ragged, verify and delta-off workloads")
    ap.add_argument("--ssd-only", action="store_true",
                    help="with --configs-only: only the delta-off (chunk 128) workload")
    ap.add_argument("--summarize-ssd-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "PASS1_DIR", "PASS2_DIR"),
                    help="summarize counter runs of SSD_PMC_CMD (FETCH_SIZE, WRITE_SIZE, the two SQ passes) "
                         "into profiles/ and exit")
    ap.add_argument("--summarize-prof", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="summarize rocprofv3 outputs of this script into profiles/ and exit")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PASS1_DIR", "PASS2_DIR"),
                    help="summarize the two SQ counter passes of PMC_CMD into profiles/ and exit")
    ap.add_argument("--summarize-configs-prof", metavar="KT_DIR",
                    help="summarize a kernel trace of the --configs-only command into profiles/ and exit")
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


def _stats_lines(kt_dir, cmd):
    lines = [f"# command (repository root): export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             f"-d <dir> -o bench -- {cmd}",
             f"# kernel sources: chunk.hip sha256 {source_sha('extend')}, recurrent.hip sha256 {source_sha('decode')}, "
             f"ssd.hip sha256 {source_sha('ssd')}, conv.hip sha256 {source_sha('conv_prefill')}",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in _csv_rows(kt_dir, "*kernel_stats.csv"):
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}  {r['Name'][:110]}")
    return lines


def summarize_configs_prof(kt_dir):
    """profiles/ summary of a kernel trace of CONFIGS_PROF_CMD: per-kernel statistics of the
    ragged extend, its verify batch and the delta-off chunk-128 call."""
    os.makedirs(PROFILES, exist_ok=True)
    lines = ["# rocprofv3 kernel-trace statistics of the ragged, verify and delta-off workloads",
             "# summarized by: python bench.py --summarize-configs-prof <kt_dir>"] + _stats_lines(kt_dir, CONFIGS_PROF_CMD)
    with open(CONFIGS_STATS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_kernel(d, counter):
    """{kernel name: [value per dispatch]} of one counter in a rocprofv3 counter run."""
    vals = {}
    for r in _csv_rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] == counter:
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _copy_scales(fetch, write):
    """FETCH_SIZE / WRITE_SIZE scale factors from the 1 GiB copy (torch.mul reads and
    writes 1 GiB): the largest MulFunctor dispatch of each run."""
    cf = max(max(v) for k, v in fetch.items() if "MulFunctor" in k)
    cw = max(max(v) for k, v in write.items() if "MulFunctor" in k)
    return cf, cw, 1024 * 1024.0 / cf, 1024 * 1024.0 / cw


def summarize_ssd_counters(fetch_dir, write_dir, dir1, dir2):
    """profiles/ summary of four counter runs of SSD_PMC_CMD: copy-scaled HBM traffic per
    dispatch of the delta-off kernels (prep, state-only pass, full pass) against the
    call's algorithmic bytes, and the two SQ counter passes with derived ratios."""
    fetch, write = _per_kernel(fetch_dir, "FETCH_SIZE"), _per_kernel(write_dir, "WRITE_SIZE")
    cf, cw, f_scale, w_scale = _copy_scales(fetch, write)
    sq = {}
    for d in (dir1, dir2):
        for r in _csv_rows(d, "*counter_collection.csv"):
            for kind, needle in SSD_KERNELS:
                if needle in r["Kernel_Name"]:
                    sq.setdefault((kind, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    lines = ["# delta-off (SSD) call at chunk 128, x [2, 8192, 80, 64]: rocprofv3 counters per dispatch",
             f"# traffic (repository root): export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- {SSD_PMC_CMD}",
             f"#   (and the same with --pmc WRITE_SIZE); KiB scaled by the copy calibration"]
    for i, counters in enumerate(SQ_PASSES):
        lines.append(f"# SQ pass {i + 1}: export TMPDIR=/tmp && rocprofv3 --pmc {' '.join(counters)} "
                     f"--output-format csv -d <dir{i + 1}> -o bench -- {SSD_PMC_CMD}")
    lines += ["# summarized by: python bench.py --summarize-ssd-counters <fetch_dir> <write_dir> <dir1> <dir2>",
              f"# kernel source: ssd.hip sha256 {source_sha('ssd')}",
              f"copy_fetch_kib {cf:.1f}", f"copy_write_kib {cw:.1f}",
              f"fetch_scale {f_scale:.4f}", f"write_scale {w_scale:.4f}"]
    total = 0
    for kind, needle in SSD_KERNELS:
        fv = [v for k, v in fetch.items() if needle in k]
        wv = [v for k, v in write.items() if needle in k]
        if not fv or not wv:
            raise SystemExit(f"kernel {needle!r} not found")
        fk, wk = sum(fv[0]) / len(fv[0]), sum(wv[0]) / len(wv[0])
        b = int(round((fk * f_scale + wk * w_scale) * 1024))
        total += b
        lines += [f"{kind}_dispatches {len(fv[0])}", f"{kind}_fetch_kib {fk:.1f}", f"{kind}_write_kib {wk:.1f}",
                  f"{kind}_traffic_bytes {b}"]
    alg = 2 * 8192 * SSD_BYTES_PER_TOKEN + 2 * SSD_H * SSD_P * SSD_N * 4
    lines += [f"call_traffic_bytes {total}", f"call_algorithmic_bytes {alg}",
              f"call_traffic_over_algorithmic {total / alg:.3f}",
              f"{'kernel':<11} {'counter':<32} {'dispatches':>10} {'avg':>12}"]
    for (kind, ctr), v in sorted(sq.items()):
        lines.append(f"{kind:<11} {ctr:<32} {len(v):10d} {sum(v) / len(v):12.4e}")
    for kind, _ in SSD_KERNELS:
        a = {ctr: sum(v) / len(v) for (k, ctr), v in sq.items() if k == kind}
        if not a:
            continue
        lines.append(f"# derived ({kind}):")
        if a.get("SQ_BUSY_CU_CYCLES"):
            lines.append(f"#   MFMA busy cycles / (busy CU cycles x 4 SIMDs): "
                         f"{a.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (4 * a['SQ_BUSY_CU_CYCLES']):.3f}")
        if a.get("SQ_ACTIVE_INST_LDS"):
            lines.append(f"#   LDS bank-conflict cycles / LDS-active cycles: "
                         f"{a.get('SQ_LDS_BANK_CONFLICT', 0) / a['SQ_ACTIVE_INST_LDS']:.2f}")
        if a.get("SQ_WAVE_CYCLES"):
            lines.append(f"#   wait cycles / wave cycles: {a.get('SQ_WAIT_ANY', 0) / a['SQ_WAVE_CYCLES']:.2f}")
        if a.get("SQ_INSTS_MFMA"):
            lines.append(f"#   VALU instructions per MFMA instruction: {a.get('SQ_INSTS_VALU', 0) / a['SQ_INSTS_MFMA']:.1f}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(SSD_COUNTERS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sq(dir1, dir2, launch_us=None):
    """profiles/ summary of the two SQ counter passes (SQ_PASSES) of PMC_CMD: the average
    per dispatch of every counter for the extend, decode and conv kernels, and derived
    ratios for the extend kernel."""
    vals = {}
    for d in (dir1, dir2):
        for r in _csv_rows(d, "*counter_collection.csv"):
            for kind in ("extend", "decode", "conv_prefill"):
                if KERNEL_NAMES[kind] in r["Kernel_Name"]:
                    vals.setdefault((kind, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    cmd = PMC_CMD
    lines = ["# SQ counters per dispatch (average over the dispatches of the profiled command)"]
    for i, counters in enumerate(SQ_PASSES):
        lines.append(f"# pass {i + 1} (repository root): export TMPDIR=/tmp && rocprofv3 --pmc {' '.join(counters)} "
                     f"--output-format csv -d <dir{i + 1}> -o bench -- {cmd}")
    lines += ["# summarized by: python bench.py --summarize-sq <dir1> <dir2>",
              f"# kernel sources: chunk.hip sha256 {source_sha('extend')}, recurrent.hip sha256 {source_sha('decode')}",
              f"{'kernel':<14} {'counter':<32} {'dispatches':>10} {'avg':>12}"]
    for (kind, ctr), v in sorted(vals.items()):
        lines.append(f"{kind:<14} {ctr:<32} {len(v):10d} {sum(v) / len(v):12.4e}")
    a = {ctr: sum(v) / len(v) for (kind, ctr), v in vals.items() if kind == "extend"}
    if a:
        lines.append("# derived (extend):")
        if a.get("SQ_BUSY_CU_CYCLES"):
            lines.append(f"#   MFMA busy cycles / (busy CU cycles x 4 SIMDs): "
                         f"{a.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (4 * a['SQ_BUSY_CU_CYCLES']):.3f}")
        mops = a.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) + a.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0)
        lines.append(f"#   MFMA FLOP from MOPS (x512): {mops * 512 / 1e9:.1f} GFLOP per dispatch")
        if a.get("SQ_ACTIVE_INST_LDS"):
            lines.append(f"#   LDS bank-conflict cycles / LDS-active cycles: "
                         f"{a.get('SQ_LDS_BANK_CONFLICT', 0) / a['SQ_ACTIVE_INST_LDS']:.2f}")
        if a.get("SQ_WAVE_CYCLES"):
            lines.append(f"#   wait cycles / wave cycles: {a.get('SQ_WAIT_ANY', 0) / a['SQ_WAVE_CYCLES']:.2f}")
        if a.get("SQ_INSTS_MFMA"):
            lines.append(f"#   VALU instructions per MFMA instruction: {a.get('SQ_INSTS_VALU', 0) / a['SQ_INSTS_MFMA']:.1f}")
    os.makedirs(PROFILES, exist_ok=True)
    with open(SQ_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_prof(kt_dir, fetch_dir, write_dir):
    """profiles/ text summaries of three rocprofv3 runs of PROF_CMD: the kernel-trace
    statistics, and FETCH_SIZE / WRITE_SIZE per dispatch scaled by what the same
    counters read for the 1 GiB copy kernel (torch.mul: reads and writes 1 GiB)."""
    os.makedirs(PROFILES, exist_ok=True)
    lines = ["# rocprofv3 kernel-trace statistics of the bench command",
             "# summarized by: python bench.py --summarize-prof <kt_dir> <fetch_dir> <write_dir>"] + _stats_lines(kt_dir, PROF_CMD)
    with open(os.path.join(PROFILES, "gdn_step_prefill_8x4096_decode_256_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fetch, write = _per_kernel(fetch_dir, "FETCH_SIZE"), _per_kernel(write_dir, "WRITE_SIZE")

    def pick(vals, needle):
        for k, v in vals.items():
            if needle in k:
                return sum(v) / len(v), len(v)
        raise SystemExit(f"kernel {needle!r} not found")
    cf, cw, f_scale, w_scale = _copy_scales(fetch, write)
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
def _cpu_unit(unit):
    """One (sequence, block of v-heads) unit of the prefill workload through the
    float64 oracle: inputs of the workload's shapes and distributions (q, k, v, a, b ~
    N(0, 1) rounded to bf16, A_log = log U(1, 16), dt_bias ~ N(0, 0.5), zero initial
    state), the whole sequence in one call.  Returns (token-heads, seconds spent in the
    oracle)."""
    seq, hb, L, hpu, seed = unit
    import numpy as np
    import oracle
    from hybrid_model_linear_amd import synth
    rng = np.random.default_rng([seed, seq, hb])
    hq = max(1, hpu // (H_V // H_QK))
    f = lambda *shape: synth.bf16_round(rng.standard_normal(shape, dtype=np.float32))
    q, k, v = f(L, hq, D), f(L, hq, D), f(L, hpu, D)
    a, b = f(L, hpu), f(L, hpu)
    A_log = np.log(rng.uniform(1.0, 16.0, hpu)).astype(np.float32)
    dt_bias = (rng.standard_normal(hpu) * 0.5).astype(np.float32)
    pool = np.zeros((1, hpu, D, D))
    t = time.perf_counter()
    oracle.gdn_extend(q, k, v, a, b, A_log, dt_bias, np.array([0, L]), np.array([0]), np.array([0]),
                      pool, D ** -0.5)
    return L * hpu, time.perf_counter() - t


def cpu_workers():
    """Worker processes for the CPU baseline: the host cores this process may run on,
    at most 16 (one GPU's share of a shared host)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def cpu_baseline(nseq=8, seqlen=4096, workers=None, seed=77):
    """The float64 oracle on the whole prefill workload (nseq sequences x seqlen tokens x
    all H_V heads) over a pool of single-threaded worker processes on the host's cores.
    A unit is one sequence with a block of its heads (the oracle is vectorised over the
    heads of a token, so whole sequences are the cheapest units; the heads are split only
    as far as needed to give every worker a unit).  tokens/s over the pool's wall time
    (input generation inside the workers included); the one-thread rate (tokens over the
    summed oracle time) is reported beside it.  Runs before anything touches the GPU
    (the workers are forked)."""
    import multiprocessing as mp
    import numpy  # noqa: F401  (imported before the fork, shared by the workers)
    import oracle  # noqa: F401
    from hybrid_model_linear_amd import synth  # noqa: F401
    workers = cpu_workers() if workers is None else workers
    hpu = H_V
    while hpu > 1 and nseq * (H_V // hpu) < workers:
        hpu //= 2
    units = [(n, hb, seqlen, hpu, seed) for n in range(nseq) for hb in range(H_V // hpu)]
    used = min(workers, len(units))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)          # one BLAS thread, inherited by the workers
    except Exception:  # pragma: no cover
        limit = None
    try:
        with mp.get_context("fork").Pool(used) as pool:
            t = time.perf_counter()
            res = pool.map(_cpu_unit, units, chunksize=1)
            wall = time.perf_counter() - t
    finally:
        if limit is not None:
            limit.__exit__(None, None, None)
    tokens = sum(r[0] for r in res) / H_V
    spent = sum(r[1] for r in res)
    return {"value": round(tokens / wall, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "host_cpus": os.cpu_count(), "one_thread_value": round(tokens / spent, 1),
            "sample": f"float64 oracle on the whole prefill workload ({nseq} sequences x {seqlen} "
                      f"tokens x {H_V} heads, zero initial states) as {len(units)} (sequence, "
                      f"{hpu}-head) units over {used} single-threaded worker processes: "
                      f"{wall:.1f} s wall, {spent:.1f} s of oracle time"}


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


def _rate(us, nbytes, flop):
    sec = us * 1e-6
    gbs, tfs = nbytes / sec / 1e9, flop / sec / 1e12
    return {"GB_s": round(gbs, 1), "TFLOP_s": round(tfs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)}


def measured_peaks(torch, gdn, reps=10):
    """The box's achievable peaks (library probes, clocks already settled): a streaming
    copy of 1 GiB (2 GiB of HBM traffic per call) and dependent chains of bf16 MFMAs
    over 8 workgroups of four waves per CU."""
    dev = "cuda"
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    us_copy = _time_calls(torch, lambda: gdn.probe_copy(src, dst), reps, warm=3, settle_ms=0.0)
    us_inplace = _time_calls(torch, lambda: gdn.probe_copy(src, src), reps, warm=3, settle_ms=0.0)
    del src, dst
    blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flop = [0]

    def mfma():
        flop[0] = gdn.probe_mfma(out, blocks, iters)
    us_mfma = _time_calls(torch, mfma, reps, warm=3, settle_ms=0.0)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("MFMA probe produced non-finite sums")
    copy, inplace = 2 * nbytes / (us_copy * 1e-6) / 1e9, 2 * nbytes / (us_inplace * 1e-6) / 1e9
    return {"copy_GB_s": round(copy, 1), "inplace_GB_s": round(inplace, 1),
            "hbm_GB_s": round(max(copy, inplace), 1),
            "mfma_bf16_TFLOP_s": round(flop[0] / (us_mfma * 1e-6) / 1e12, 1),
            "copy": "gdn_probe_copy, 1 GiB read and 1 GiB written: into another buffer (copy) and "
                    "back into itself (in place, the decode's state pattern); hbm_GB_s the larger",
            "mfma": f"gdn_probe_mfma, {blocks} workgroups x 4 waves x 4 chains x {iters} "
                    "32x32x16 bf16 MFMAs"}


def _time_calls(torch, fn, steps, warm=10, settle_ms=100.0):
    """Average microseconds per call of fn over `steps` back-to-back calls, from HIP events
    recorded on torch's current stream (the stream the calls launch on), after at least
    `warm` calls and `settle_ms` of back-to-back calls (clocks settled)."""
    n, t0 = 0, time.time()
    while n < warm or (time.time() - t0) * 1e3 < settle_ms:
        fn()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


SSD_H, SSD_P, SSD_N, SSD_G, SSD_CHUNK = 80, 64, 128, 1, 128
SSD_BYTES_PER_TOKEN = 3 * SSD_H * SSD_P * 2 + SSD_H * 2 + 2 * SSD_G * SSD_N * 2   # x, z, out; dt; B, C
SSD_FLOP_PER_TOKEN = SSD_H * 2 * (SSD_CHUNK * SSD_P + 2 * SSD_N * SSD_P) + 2 * SSD_CHUNK * SSD_N * SSD_G


def bench_configs(torch, gdn, synth, steps, only=None):
    """The other workloads, each timed on its own (not part of the step): the ragged
    extend from pooled states (64 sequences, ~131k tokens) and its verify batch (32 x 4
    tokens), and the delta-off (SSD) call at chunk 128 (x [2, 8192, 80, 64]).  Inputs
    resident in HBM; outputs, pools and the delta-off workspace allocated before timing."""
    dev = "cuda"
    t32 = lambda x: torch.from_numpy(x).to(dev, torch.float32)
    ti = lambda x: torch.from_numpy(x).to(dev, torch.int32)
    res = {}

    def gdn_leg(case, pool, max_seqlen):
        q, k, v = gdn.split_mixed_qkv(case.mixed_qkv, case.H_qk, case.H_v, case.d_k, case.d_v)
        g = gdn.gdn_gate_inputs(case.a, case.b, t32(case.A_log), t32(case.dt_bias))
        out = torch.empty((case.T, case.H_v, case.d_v), dtype=torch.bfloat16, device=dev)
        cu, slot, hi = ti(case.cu_seqlens), ti(case.slot), ti(case.has_init)
        kern = gdn.extend_kernel(q, k, v, None, None, cu, slot, pool, has_init=hi, scale=case.scale,
                                 max_seqlen=max_seqlen, gate=g)
        fn = lambda: gdn.extend(q, k, v, None, None, cu, slot, pool, has_init=hi, scale=case.scale,
                                out=out, max_seqlen=max_seqlen, gate=g)
        return _time_calls(torch, fn, steps), kern

    # ragged extend from pooled states, then its verify batch on other slots of the pool
    if only is not None and "ssd_chunk128" in only:
        return {"ssd_chunk128": bench_ssd(torch, gdn, synth, steps)}
    rag = synth.device_config3_ragged()
    pool3 = synth.device_pool(rag)
    lens = rag.cu_seqlens[1:] - rag.cu_seqlens[:-1]
    us, kern = gdn_leg(rag, pool3, int(lens.max()))
    nbytes = rag.T * IO_BYTES_PER_TOKEN + rag.N * 2 * STATE_BYTES        # states read and written
    flop = rag.T * EXTEND_FLOP_PER_TOKEN
    res["ragged_extend"] = dict(workload=f"extend {rag.N} ragged sequences (log-uniform lengths "
                                         f"{int(lens.min())}..{int(lens.max())}, {rag.T} tokens) from "
                                         f"pooled states, pool [512,32,128,128] fp32",
                                kernel=kern[0], avg_us=round(us, 2), tokens_per_s=round(rag.T / (us * 1e-6), 1),
                                bytes=nbytes, flop=flop, **_rate(us, nbytes, flop))
    ver = synth.device_config3_verify()
    us, kern = gdn_leg(ver, pool3, 4)
    nbytes = ver.T * IO_BYTES_PER_TOKEN + ver.N * 2 * STATE_BYTES
    flop = ver.T * 7 * H_V * D * D
    res["verify_extend"] = dict(workload="extend 32 sequences x 4 tokens from pooled states",
                                kernel=kern[0], avg_us=round(us, 2), tokens_per_s=round(ver.T / (us * 1e-6), 1),
                                bytes=nbytes, flop=flop, **_rate(us, nbytes, flop))
    del rag, ver, pool3
    res["ssd_chunk128"] = bench_ssd(torch, gdn, synth, steps)
    return res


def bench_ssd(torch, gdn, synth, steps):
    """The delta-off (Mamba2 SSD) call at chunk 128 on x [2, 8192, 80, 64]."""
    dev = "cuda"
    c = synth.device_config4_ssd()
    batch, L = c.x.shape[0], c.x.shape[1]
    T = batch * L
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device=dev)
    slot = torch.arange(batch, dtype=torch.int32, device=dev)
    hi = torch.zeros(batch, dtype=torch.int32, device=dev)
    pool = torch.zeros((batch, SSD_H, SSD_P, SSD_N), dtype=torch.float32, device=dev)
    out = torch.empty((T, SSD_H, SSD_P), dtype=torch.bfloat16, device=dev)
    g = gdn.ssd_gate_inputs(c.dt.view(T, SSD_H), c.A, c.dt_bias, True, (0.0, float("inf")))
    qkv = (c.C.view(T, SSD_G, SSD_N), c.B.view(T, SSD_G, SSD_N), c.x.view(T, SSD_H, SSD_P))
    kw = dict(has_init=hi, mode="ssd", D=c.D, z=c.z.view(T, SSD_H, SSD_P), max_seqlen=L, gate=g)
    need = gdn.extend_workspace_size(*qkv, None, None, cu, slot, pool, **kw)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    kern = gdn.extend_kernel(*qkv, None, None, cu, slot, pool, workspace=ws, **kw)
    us = _time_calls(torch, lambda: gdn.extend(*qkv, None, None, cu, slot, pool, out=out, workspace=ws, **kw),
                     steps)
    nbytes = T * SSD_BYTES_PER_TOKEN + batch * SSD_H * SSD_P * SSD_N * 4   # zero init: states written
    flop = T * SSD_FLOP_PER_TOKEN
    return dict(workload=f"delta-off (SSD) x [{batch},{L},{SSD_H},{SSD_P}], B/C [{batch},{L},{SSD_G},{SSD_N}], "
                         f"D, silu(z), chunk 128, zero initial states", kernel=kern[0], workspace_bytes=int(need),
                avg_us=round(us, 2), tokens_per_s=round(T / (us * 1e-6), 1), bytes=nbytes, flop=flop,
                **_rate(us, nbytes, flop))


def main():
    args = parse()
    if args.summarize_prof:
        summarize_prof(*args.summarize_prof)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq)
        return
    if args.summarize_configs_prof:
        summarize_configs_prof(args.summarize_configs_prof)
        return
    if args.summarize_ssd_counters:
        summarize_ssd_counters(*args.summarize_ssd_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer needs no collective; heads and "
              f"sequences shard independently); --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)
    cpu = None
    if not args.no_cpu_baseline:   # (before anything touches the GPU: its workers are forked)
        print(f"[bench] timing the CPU oracle baseline on {cpu_workers()} worker(s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
        print(f"[bench] CPU oracle baseline: {cpu['value']} tokens/s", file=sys.stderr, flush=True)
    import torch
    import hybrid_model_linear_amd as gdn
    from hybrid_model_linear_amd import synth

    gdn.load()
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.configs_only:
        if args.calibrate_copy_mib:   # (counter scaling, as in the step's profile)
            src = torch.ones((args.calibrate_copy_mib << 20) // 4, dtype=torch.float32, device=dev)
            torch.mul(src, 1.0, out=torch.empty_like(src))
            torch.cuda.synchronize()
            del src
        only = ("ssd_chunk128",) if args.ssd_only else None
        print(json.dumps({"configs": bench_configs(torch, gdn, synth, args.steps, only=only)}), flush=True)
        return
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

    settle_steps, t0 = 0, time.time()
    while (time.time() - t0) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    settle_ms = (time.time() - t0) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] clocks settled ({settle_steps} steps, {settle_ms:.0f} ms); warmup done "
          f"({args.warmup} steps)", file=sys.stderr, flush=True)

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
    peaks = measured_peaks(torch, gdn)
    for n in names:   # against the box's measured peaks as well as the published ones
        kernels[n]["hbm_frac_measured"] = round(kernels[n]["GB_s"] / peaks["hbm_GB_s"], 4)
        kernels[n]["mfma_frac_measured"] = round(kernels[n]["TFLOP_s"] / peaks["mfma_bf16_TFLOP_s"], 4)
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
                "mfma_frac": kd["mfma_frac"], "avg_launch_us": kd["avg_us"],
                "frac_of_measured_peak": kd["hbm_frac_measured"] if ai < ridge else kd["mfma_frac_measured"]}
    tokens = T_e + T_d
    result = {
        "metric": METRIC, "value": round(tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps},
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
        "measured_peaks": peaks,
    }
    result["conv1d"] = bench_conv(torch, gdn, T_e, ext.N, T_d, args.steps)
    if not args.no_configs:
        print("[bench] ragged, verify and delta-off workloads", file=sys.stderr, flush=True)
        result["configs"] = bench_configs(torch, gdn, synth, args.steps)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
