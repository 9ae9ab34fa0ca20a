"""Decode-step benchmark on one MI355X: tokens/s and achieved HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one qd_decode_step call (timed as a HIP-graph replay of that call,
captured once; the eager-launch rate is reported beside it): embedding, every layer (fused RMSNorm + QKV
GEMV, q/k norm + RoPE + KV append, split-K attention + merge, o_proj + residual,
RMSNorm + gate/up + SwiGLU, down + residual), final norm, lm_head and greedy
argmax, for one batch of synthetic input already resident in HBM. Each step
re-runs the same positions (the step is idempotent at a position), so every
timed step attends over exactly `past` cached tokens.

The K timed steps run in rounds that alternate with rounds of the CPU oracle
(when the CPU baseline is on), each GPU round after a few untimed replays;
`value` is all timed steps over their summed time. Per-step times (an event
between consecutive replays, in a separate pass) give the median, minimum and
spread. A 1 GiB device copy at the start and at the end of the run is the
HBM thermometer.

Prints ONE JSON line. `roofline` covers the dominant kernel kind: its
algorithmic bytes per launch divided by its average launch duration. The
duration is taken from a rocprofv3 kernel trace of a child run of the same
workload (same graph replays), started before this process touches the GPU,
so it is the figure a `rocprofv3 --kernel-trace --stats` summary of this
command reports; when rocprofv3 is not available, from HIP events around each
launch (net of an event pair's own cost, plus an equal share of the replayed
step's dispatch time). `traffic` is the measured HBM bytes per launch of that
kernel from the hardware-counter summaries under profiles/, when they were
taken from the current sources.
`cpu_baseline` is the fp64 oracle timed on the host over a bounded sample of
whole decode steps of the same workload, with the machine it ran on, its
thread count and a single-thread figure.
Every run appends its record, with the per-step samples, the machine, the
versions and the source revision, to an append-only log (--log).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode tokens/s + achieved HBM GB/s (% of peak), Qwen2-0.5B-shape, batch 1/16"


def _dtype_bytes(shape):
    """(bytes per matrix element, extra bytes per matrix row, bytes per gain or bias
    element): int8 matrices carry a float32 scale per row and bf16 gains/biases."""
    if shape.w_dtype == "i8":
        return 1, 4, 2
    wb = 2 if shape.w_dtype == "bf16" else 4
    return wb, 0, wb


def _bytes_per_launch(shape, B, ctx):
    """Algorithmic bytes per launch of each kernel kind: weights read once, KV read
    once, activations counted at their float32 size."""
    from decode_step_amd import qd as Q
    from decode_step_amd.runner import make_config
    wb, rb, gb = _dtype_bytes(shape)
    kvb = 2 if shape.kv_dtype == "bf16" else 4
    D, F, V = shape.hidden, shape.ffn, shape.vocab
    qd_, kvd = shape.q_dim, shape.kv_dim
    qkvr = qd_ + 2 * kvd
    kv_tokens = int(np.sum(ctx + 1))
    act = 4
    out = {
        Q.QD_K_QKV: qkvr * (D * wb + rb) + (qkvr * gb if shape.qkv_bias else 0) + D * gb + B * (D + qkvr) * act,
        Q.QD_K_ATTN: kv_tokens * 2 * kvd * kvb + B * qd_ * act,
        Q.QD_K_O: D * (qd_ * wb + rb) + B * (qd_ + 2 * D) * act,
        Q.QD_K_GATEUP: 2 * F * (D * wb + rb) + D * gb + B * (D + F) * act,
        Q.QD_K_DOWN: D * (F * wb + rb) + B * (F + 2 * D) * act,
        Q.QD_K_LMHEAD: V * (D * wb + rb) + D * gb + B * (D + V) * act,
    }
    # batch 1 with the projection inside the attention launch: that launch also moves
    # the projection's bytes (q|k|v rows, biases, gain, x, the projected vectors)
    if B == 1 and Q.qd_decode_plan(make_config(shape), 1, int(np.max(ctx)) + 1).fused_qkv:
        out[Q.QD_K_ATTN] += out.pop(Q.QD_K_QKV)
    return out


def step_bytes(shape, B, ctx, block_only=False):
    """Algorithmic bytes of one whole step (every weight once, every cached K/V once,
    the new K/V written, the embedding rows and the logits); block_only: the decoder
    blocks alone (their matrices, gains and biases, the K/V, the float32 vector in
    and out)."""
    wb, rb, gb = _dtype_bytes(shape)
    kvb = 2 if shape.kv_dtype == "bf16" else 4
    c = shape.param_counts()
    D, F, V, L = shape.hidden, shape.ffn, shape.vocab, shape.n_layers
    # matrices (and their rows), then norm gains and biases; every parameter once,
    # except that an untied embedding table is only gathered (B rows, counted below);
    # a tied table is read whole as the lm_head
    bias = L * (shape.q_dim + 2 * shape.kv_dim) if shape.qkv_bias else 0
    mat = c["total"] - c["norms"] - bias - (0 if shape.tied else V * D)
    rows = L * (shape.q_dim + 2 * shape.kv_dim + D + 2 * F + D) + V
    weights = mat * wb + rows * rb + (c["norms"] + bias) * gb
    kv_read = int(np.sum(ctx)) * shape.n_layers * 2 * shape.kv_dim * kvb
    kv_write = B * shape.n_layers * 2 * shape.kv_dim * kvb
    if block_only:
        # mat holds one vocabulary table (the lm_head, or the tied table read as one),
        # rows its row scales, norms the final norm
        blocks = (mat - V * D) * wb + (rows - V) * rb + (c["norms"] - D + bias) * gb
        return blocks + kv_read + kv_write + 2 * B * D * 4
    emb_rows = B * (D * wb + rb)
    logits = B * shape.vocab * 4
    return weights + kv_read + kv_write + emb_rows + logits


def csrc_digest():
    """sha256 over the HIP sources of libqd (file names and contents, sorted): the
    hardware-counter figures under profiles/ hold only for the sources they were
    taken from."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decode_step_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch of `kernel` from the FETCH_SIZE / WRITE_SIZE counter
    summaries in profiles/ (lines 'traffic: {json}'), or None when none was taken
    for these exact sources."""
    import glob
    digest = csrc_digest()
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(f) as fh:
            for line in fh:
                if not line.startswith("traffic: "):
                    continue
                rec = json.loads(line[len("traffic: "):])
                if rec.get("workload") == workload and rec.get("kernel") == kernel:
                    if rec.get("csrc_sha256") == digest:
                        return int(rec["bytes_per_launch"]), os.path.relpath(f, ROOT)
                    return None, f"{os.path.relpath(f, ROOT)} (taken from other sources)"
    return None, "no counter run for these sources"


def machine_info() -> dict:
    """The host this run is on: CPU model, logical CPUs and those this process may use."""
    import socket
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return {"host": socket.gethostname(), "cpu_model": model, "nproc": os.cpu_count() or 1,
            "cpus_allowed": allowed}


def versions_info(torch) -> dict:
    """Source revision and the software stack of the run."""
    import subprocess
    sha = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        sha = r.stdout.strip() or None
    except Exception:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as fh:
            rocm = fh.read().strip()
    except OSError:
        pass
    return {"git": sha, "csrc_sha256": csrc_digest(), "torch": torch.__version__, "hip": torch.version.hip,
            "rocm": rocm, "python": sys.version.split()[0], "numpy": np.__version__}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def hbm_probe(torch, nbytes=1 << 30, reps=3) -> float:
    """GB/s (read + write) of a plain device copy of nbytes, reps times: a
    thermometer for the HBM and clocks at the start and end of a run."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del src, dst
    return round(2 * nbytes * reps / el / 1e9, 1)


# kernel names of each kind (the demangled names a rocprofv3 kernel trace reports)
KIND_KERNELS = {
    "gate_up_gemv": [r"gemv1_kernel<[^>]*, 2, \d+>\(", r"gemm16_rows_kernel<"],
    "lm_head_gemv": [r"gemv1_kernel<[^>]*, 3, \d+>\(", r"gemm16_kernel<3,"],
    "down_gemv": [r"gemv1_kernel<[^>]*, 10, 1, 0>\(", r"gemm16_split_kernel<1, 5,"],
    "attention": [r"attn_kernel<", r"attn_mfma_kernel<", r"attn_fq_kernel<"],
    "step_kernel": [r"step_kernel\("],
}


def trace_child(args, n_steps):
    """Average kernel durations of a child run of this workload under rocprofv3
    (--kernel-trace --stats): the same graph replays as the timed region. Runs
    before this process touches the GPU. Returns {kernel name: (calls, avg us)}
    or None (rocprofv3 missing or the run failed)."""
    import shutil
    import subprocess
    import tempfile
    import csv
    prof = shutil.which("rocprofv3") or ("/opt/rocm/bin/rocprofv3" if os.path.exists("/opt/rocm/bin/rocprofv3")
                                         else None)
    if prof is None:
        return None, "rocprofv3 not found"
    with tempfile.TemporaryDirectory(prefix="qd_trace_") as tmp:
        cmd = [prof, "--kernel-trace", "--stats", "-d", tmp, "-o", "rp", "--output-format", "csv", "--",
               sys.executable, os.path.abspath(__file__), "--workload", args.workload, "--steps", str(n_steps),
               "--warmup", str(min(args.warmup, 20)), "--trace-child"]
        env = dict(os.environ)
        env.setdefault("TMPDIR", "/tmp")
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, env=env, cwd=ROOT)
        except Exception as e:   # noqa: BLE001 (any failure leaves the event figure)
            return None, f"rocprofv3 child failed: {e}"
        path = os.path.join(tmp, "rp_kernel_stats.csv")
        if not os.path.exists(path):
            return None, f"rocprofv3 child left no kernel stats (exit {r.returncode})"
        out = {}
        with open(path) as fh:
            for row in csv.DictReader(fh):
                out[row["Name"]] = (int(row["Calls"]), float(row["AverageNs"]) / 1e3)
        return out, " ".join(cmd[:8] + ["--", "python3", "bench.py", "--workload", args.workload,
                                        "--steps", str(n_steps), "--trace-child"])


def kind_duration(stats, kind):
    """Call-weighted average duration (us) of the kernels of one kind in a trace."""
    import re
    pats = KIND_KERNELS.get(kind, [])
    calls, tot = 0, 0.0
    for name, (n, avg) in stats.items():
        if any(re.search(p, name) for p in pats):
            calls += n
            tot += n * avg
    return (tot / calls, calls) if calls else (None, 0)


class OracleTimer:
    """The fp64 oracle's whole decode steps on the host, timed in rounds that
    alternate with the GPU's, plus a single-thread figure."""

    def __init__(self, wl, case_host, ctx, tokens, x_in=None):
        from oracle.qwen2 import OracleWeights, decode_step
        self.decode_step = decode_step
        self.wl, self.ctx, self.tokens, self.x_in = wl, ctx, tokens, x_in
        self.host_w, self.kh, self.vh, self.table = case_host
        self.ow = OracleWeights(wl.shape, self.host_w, cache_layers=True)
        self.threads = blas_threads()
        self.one()                       # untimed: widens the weights
        self.steps, self.secs, self.rounds = 0, 0.0, []

    def one(self):
        if self.x_in is not None:   # one decoder block from the float32 vector
            self.decode_step(self.wl.shape, self.ow, self.kh, self.vh, self.table, self.ctx, x_in=self.x_in,
                             with_logits=False)
        else:
            self.decode_step(self.wl.shape, self.ow, self.kh, self.vh, self.table, self.ctx, tokens=self.tokens)

    def round(self, budget_s):
        n, t0 = 0, time.perf_counter()
        while True:
            self.one()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or el > 4 * budget_s:
                break
        self.steps += n
        self.secs += el
        self.rounds.append(round(len(self.ctx) * n / el, 4))

    def single_thread(self, budget_s):
        try:
            from threadpoolctl import threadpool_limits
        except Exception:
            return None
        with threadpool_limits(limits=1):
            n, t0 = 0, time.perf_counter()
            while True:
                self.one()
                n += 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
        B = len(self.ctx)
        return {"value": round(B * n / el, 4), "unit": "tokens/s", "threads": 1,
                "sample": f"{n} whole decode steps in {el:.1f} s with BLAS limited to one thread"}

    def record(self, single):
        B = len(self.ctx)
        m = machine_info()
        return {"value": round(B * self.steps / self.secs, 4), "unit": "tokens/s", "cores": int(self.threads),
                "kind": "oracle",
                "sample": f"{self.steps} whole decode steps of {self.wl.name} (batch {B}) in {self.secs:.1f} s over "
                          f"{len(self.rounds)} rounds alternating with the GPU's, fp64 numpy, after one untimed "
                          f"step that widens the weights",
                "threads": int(self.threads), "cpu_model": m["cpu_model"], "nproc": m["nproc"],
                "cpus_allowed": m["cpus_allowed"], "rounds": self.rounds, "single_thread": single}


def append_log(path, entry):
    """Append one JSON line to the run log (created with its folder if missing)."""
    if not path:
        return
    try:
        d = os.path.dirname(os.path.abspath(path))
        os.makedirs(d, exist_ok=True)
        with open(path, "a") as fh:
            fh.write(json.dumps(entry) + "\n")
    except OSError as e:
        print(f"[bench] could not append to {path}: {e}", file=sys.stderr)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(shape, n, start=0):
    """2*M*N*K over the four projection GEMMs, and the causal attention's
    2 * Hq * hd * (sum over rows of keys attended) * 2 (scores and P.V)."""
    D, F, qd, kvd = shape.hidden, shape.ffn, shape.q_dim, shape.kv_dim
    gemm = 2 * n * ((qd + 2 * kvd) * D + D * qd + 2 * F * D + D * F)
    keys = sum(start + i + 1 for i in range(n))
    attn = 2 * shape.n_q_heads * shape.head_dim * keys * 2
    return gemm, attn


def bench_prefill(wl, args):
    import torch
    from decode_step_amd import qd as Q
    from decode_step_amd.runner import DecodeRunner
    from workloads import synth
    sh, n = wl.shape, wl.prefill_tokens
    w = synth.make_weights(sh, seed=wl.seed, device="cuda", with_embed=False)
    kv = synth.make_kv(sh, np.array([0]), extra=n, seed=wl.seed, device="cuda")
    runner = DecodeRunner(sh, w, kv.k, kv.v, kv.block_table, max_batch=1, max_ctx=n, device="cuda",
                          prefill_tokens=n)
    x = synth.make_x(n, sh.hidden, seed=wl.seed, dtype="bf16", device="cuda")
    x_out = torch.empty(n, sh.hidden, device="cuda")

    def step():
        runner.prefill(0, n, 0, x, x_out, stream=torch.cuda.current_stream())

    for _ in range(args.warmup):
        step()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    probe_start = hbm_probe(torch)
    # the oracle's block on a bounded sample: the first n_s rows of the same block
    # (the GEMM work per row is the same; each row attends over fewer keys)
    oracle = None
    if not args.no_cpu_baseline:
        from oracle.qwen2 import OracleWeights, prefill_block
        host_w = synth.weights_to_host(w)
        W = OracleWeights(sh, host_w, cache_layers=False).layer(0)
        n_s = min(n, 32)
        X = synth.to_host_bits(x[:n_s])
        pools = (synth.to_host_bits(kv.k[0]).copy(), synth.to_host_bits(kv.v[0]).copy())
        oracle = {"W": W, "X": X, "n_s": n_s, "rows": 0, "secs": 0.0, "rounds": []}

        def oracle_round(budget_s):
            c, t0 = 0, time.perf_counter()
            while True:
                prefill_block(sh, oracle["W"], pools[0], pools[1], kv.block_table[0], 0, oracle["X"])
                c += 1
                el_ = time.perf_counter() - t0
                if el_ >= budget_s:
                    break
            oracle["rows"] += c * n_s
            oracle["secs"] += el_
            oracle["rounds"].append(round(c * n_s / el_, 3))
    R = max(1, min(args.rounds, args.steps))
    per = [args.steps // R + (1 if r < args.steps % R else 0) for r in range(R)]
    el = 0.0
    for r in range(R):
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(per[r]):
            graph.replay()
        torch.cuda.synchronize()
        el += time.perf_counter() - t0
        if oracle is not None:
            oracle_round(15.0 / R)
    gemm_f, attn_f = prefill_flops(sh, n)
    ms = 1e3 * el / args.steps
    # profiled pass: GEMM launches and attention
    Q.qd_profile_enable((1 << Q.QD_K_PREFILL_GEMM) | (1 << Q.QD_K_PREFILL_ATTN))
    np_ = min(args.steps, 200)
    for _ in range(np_):
        step()
    torch.cuda.synchronize()
    ng, ms_g = Q.qd_profile_read(Q.QD_K_PREFILL_GEMM)
    na, ms_a = Q.qd_profile_read(Q.QD_K_PREFILL_ATTN)
    Q.qd_profile_enable(0)
    gemm_s = ms_g * 1e-3 / np_          # every GEMM launch of one block (with the down slabs' sum)
    gemm_tfs = gemm_f / gemm_s / 1e12
    print(f"[bench] {wl.name}: {ms:.4f} ms/block, GEMMs {1e6 * gemm_s:.1f} us = {gemm_tfs:.1f} TFLOP/s "
          f"({100 * gemm_tfs / MFMA_BF16_PEAK_TFLOPS:.1f}% of bf16 MFMA peak), attention "
          f"{1e3 * ms_a / np_:.1f} us", file=sys.stderr, flush=True)
    rec = {"metric": "prefill tokens/s + bf16 MFMA utilisation, 8B-shape block, 512 tokens",
           "value": round(n * args.steps / el, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "tokens": n, "start": 0}, "launch": "hip_graph",
           "block_tflops": round((gemm_f + attn_f) / el * args.steps / 1e12, 1),
           "roofline": {"bound": "mfma", "achieved": round(gemm_tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(gemm_tfs / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": f"mfma_gemm ({ng // np_} launches per block: q|k|v, o_proj, gate|up, down"
                                  f"{', the sum of the down K ranges' if ng // np_ > 4 else ''})",
                        "flops_per_block": int(gemm_f),
                        "avg_block_gemm_us": round(1e6 * gemm_s, 2)},
           "attention_us": round(1e3 * ms_a / np_, 2), "cpu_baseline": None,
           "hbm_probe_gbs": {"start": probe_start, "end": hbm_probe(torch),
                             "what": "1 GiB device copy x3, read + write"},
           "gpu": torch.cuda.get_device_name(0), "machine": machine_info()}
    if oracle is not None:
        m = machine_info()
        rec["cpu_baseline"] = {
            "value": round(oracle["rows"] / oracle["secs"], 3), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{oracle['rows'] // oracle['n_s']} oracle prefill_block calls over the first "
                      f"{oracle['n_s']} rows of the same block ({oracle['rows']} rows in {oracle['secs']:.1f} s, "
                      f"{len(oracle['rounds'])} rounds alternating with the GPU's), fp64 numpy; rows attend "
                      f"over fewer keys than the full block's average",
            "threads": blas_threads(), "cpu_model": m["cpu_model"], "nproc": m["nproc"],
            "cpus_allowed": m["cpus_allowed"], "rounds": oracle["rounds"]}
    print(json.dumps(rec), flush=True)
    append_log(args.log, {"time": time.strftime("%Y-%m-%dT%H:%M:%S%z"), "argv": sys.argv[1:], "record": rec,
                          "versions": versions_info(torch)})


COPY_PROBE_BYTES = 1 << 30


def copy_probe(reps=5):
    """A plain copy of COPY_PROBE_BYTES between two device buffers, reps times:
    each launch reads and writes exactly that many bytes, so the hardware
    counters it reads give the scale from counter units to bytes."""
    import torch
    src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "reps": reps,
                      "gbs_read_plus_write": round(2 * COPY_PROBE_BYTES * reps / el / 1e9, 1)}), flush=True)


def bench_sample(wl, args):
    """qd_sample over B rows of seeded logits, timed over K back-to-back launches."""
    import torch
    from decode_step_amd.runner import sample
    from workloads import synth
    B, V, X = wl.batch, wl.shape.vocab, wl.extra
    logits = synth.normal((B, V), X["logit_std"], 0.0, "f32", wl.seed, "sample_logits", "cuda")
    u = torch.from_numpy(synth.uniform_int(B, 0, (1 << 24) - 1, wl.seed, "sample_u").astype(np.float32)
                         / float(1 << 24)).cuda()
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    run = lambda: sample(logits, X["temperature"], X["top_k"], X["top_p"], u, tok)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / args.steps
    nbytes = B * V * 4                     # every logit read once
    gbs = nbytes / (us * 1e-6) / 1e9
    print(f"[bench] {wl.name}: {us:.2f} us per call ({B} rows), {gbs:.1f} GB/s of logits", file=sys.stderr)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle.sampler import sample as oracle_sample
        lh, uh = logits.cpu().numpy(), u.cpu().numpy()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0 or n < 1:
            oracle_sample(lh, X["temperature"], X["top_k"], X["top_p"], uh)
            n += 1
        el = time.perf_counter() - t0
        m = machine_info()
        cpu = {"value": round(B * n / el, 2), "unit": "sampled tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} calls of the numpy oracle sampler over the same {B} x {V} logits in {el:.1f} s "
                         f"(numpy sorts and cumulative sums: one thread)",
               "threads": 1, "cpu_model": m["cpu_model"], "nproc": m["nproc"], "cpus_allowed": m["cpus_allowed"]}
    rec = {"metric": "sampled tokens/s, temperature/top-k/top-p sampler, 0.5B vocabulary",
           "value": round(B / (us * 1e-6), 1), "unit": "sampled tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": wl.name, "batch": B, "vocab": V, **X}, "launch": "eager",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "sample_kernel",
                        "bytes_per_launch": nbytes, "avg_launch_us": round(us, 3)},
           "gpu": torch.cuda.get_device_name(0), "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)
    append_log(args.log, {"time": time.strftime("%Y-%m-%dT%H:%M:%S%z"), "argv": sys.argv[1:], "record": rec,
                          "versions": versions_info(torch)})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen2-0.5b-bf16-b1-past512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--no-trace-child", action="store_true",
                    help="take the dominant kernel's duration from HIP events instead of a rocprofv3 child run "
                         "(use when this command itself runs under rocprofv3)")
    ap.add_argument("--trace-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--rounds", type=int, default=3, help="GPU / CPU-oracle rounds that alternate")
    ap.add_argument("--rotate", type=int, default=0,
                    help="weight copies the steps rotate through, so that each step streams its weights from "
                         "HBM rather than the last-level cache (default: 24 for a one-block workload, else 1)")
    ap.add_argument("--log", default=os.path.join(ROOT, "results", "bench_runs.jsonl"),
                    help="append-only JSON-lines log of every run ('' for none)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device-to-device copy of 1 GiB (5 times): the reference kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the decode step runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding over several GPUs is a design, not an implemented path.", file=sys.stderr)
        sys.exit(2)

    from workloads import shapes as S
    wl = S.WORKLOADS[args.workload]
    # the kernel trace of a child run comes first, before this process initialises the GPU
    trace, trace_src = None, "events (--no-trace-child)"
    if wl.kind == "decode" and not args.trace_child and not args.no_trace_child and not args.copy_probe:
        trace, trace_src = trace_child(args, min(args.steps, 100))

    import torch
    from decode_step_amd import qd as Q
    from decode_step_amd.runner import DecodeRunner
    from workloads import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        return copy_probe()
    if wl.kind == "prefill":
        return bench_prefill(wl, args)
    if wl.kind == "sample":
        return bench_sample(wl, args)
    shape = wl.shape
    dev = "cuda"
    probe_start = None if args.trace_child else hbm_probe(torch)
    ctx = synth.make_ctx(wl.batch, wl.past, wl.ctx_range, wl.seed)
    B = wl.batch
    w = synth.make_weights(shape, seed=wl.seed, device=dev)
    host_w = None
    if shape.w_dtype == "i8":   # the bf16 draw through the library's int8 quantizer
        from decode_step_amd.runner import quantize_weights_int8
        if not args.no_cpu_baseline:
            host_w = synth.weights_to_host(w)
        w = quantize_weights_int8(w)
        torch.cuda.synchronize()
    kv = synth.make_kv(shape, ctx, extra=2, seed=wl.seed, device=dev, random_order=wl.paged_random)
    # weight copies the steps rotate through (the blocks' tensors only; the vocabulary
    # tables are shared): a one-block workload's weights (60 MB in fp32 for the 0.5B
    # block) fit the last-level cache, so one copy would time cache hits, not HBM
    rotate = args.rotate if args.rotate > 0 else (24 if wl.block_only else 1)
    w_copies = [w] + [{**w, "layers": [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in L.items()}
                                       for L in w["layers"]]} for _ in range(rotate - 1)]
    runners = [DecodeRunner(shape, wr, kv.k, kv.v, kv.block_table, max_batch=B, max_ctx=int(ctx.max()) + 2,
                            device=dev) for wr in w_copies]
    runner = runners[0]
    tokens = synth.make_tokens(B, shape.vocab, seed=wl.seed, name="tok0")
    tok_d = torch.from_numpy(tokens).to(dev)
    pos_d = torch.from_numpy(ctx).to(dev)
    logits = torch.empty(B, shape.vocab, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    x_in = synth.make_x(B, shape.hidden, seed=wl.seed, device=dev) if wl.block_only else None
    x_out = torch.empty(B, shape.hidden, device=dev) if wl.block_only else None
    turn = [0]

    def step_with(r):
        if wl.block_only:   # one decoder block: the float32 vector in and out
            r.step(ctx, pos_d, x_in=x_in, x_out=x_out, stream=torch.cuda.current_stream())
        else:
            r.step(ctx, pos_d, tokens=tok_d, logits=logits, next_tokens=nxt, stream=torch.cuda.current_stream())

    def step():
        step_with(runners[turn[0] % rotate])
        turn[0] += 1

    def timed(fn, k):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def capture():
        """One graph per weight copy; the returned call replays them in turn."""
        graphs = []
        for r in runners:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step_with(r)
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_with(r)
            graphs.append(g)

        def replay():
            graphs[turn[0] % rotate].replay()
            turn[0] += 1
        return replay

    if args.trace_child:   # the replays a rocprofv3 parent traces, nothing else
        for _ in range(args.warmup):
            step()
        replay = capture()
        for _ in range(args.warmup):
            replay()
        timed(replay, args.steps)
        return

    sb = step_bytes(shape, B, ctx, block_only=wl.block_only)
    # eager launches (one qd_decode_step call per step)
    for _ in range(args.warmup):
        step()
    el_eager = timed(step, args.steps)
    print(f"[bench] {wl.name} eager: {1e3 * el_eager / args.steps:.4f} ms/step, "
          f"{B * args.steps / el_eager:.1f} tokens/s", file=sys.stderr, flush=True)
    # the same call captured once in a HIP graph and replayed
    graph = None if args.no_graph else capture()
    run = graph if graph else step
    for _ in range(args.warmup):
        run()

    # the CPU oracle, set up before the rounds so that its rounds alternate with the GPU's
    oracle = None
    if not args.no_cpu_baseline:
        if shape.w_dtype == "i8":   # the oracle runs the same codes dequantized
            from oracle.quant import quantized_model
            hw = quantized_model(host_w)[0]
        else:
            hw = synth.weights_to_host(w)
        case_host = (hw, [synth.to_host_bits(t).copy() for t in kv.k],
                     [synth.to_host_bits(t).copy() for t in kv.v], kv.block_table)
        oracle = OracleTimer(wl, case_host, ctx, tokens,
                             x_in=synth.to_host_bits(x_in).astype(np.float64) if wl.block_only else None)

    # timed rounds: K steps split over R rounds, each after 3 untimed replays, with
    # an oracle round after each GPU round
    R = max(1, min(args.rounds, args.steps))
    per = [args.steps // R + (1 if r < args.steps % R else 0) for r in range(R)]
    elapsed, gpu_rounds = 0.0, []
    for r in range(R):
        for _ in range(3):
            run()
        el = timed(run, per[r])
        elapsed += el
        gpu_rounds.append(round(B * per[r] / el, 2))
        if oracle is not None:
            oracle.round(12.0 / R)
    ms_per_step = 1e3 * elapsed / args.steps
    tok_s = B * args.steps / elapsed
    print(f"[bench] {wl.name} {'graph' if graph else 'eager'}: {ms_per_step:.4f} ms/step, {tok_s:.1f} tokens/s, "
          f"{sb / 1e6:.2f} MB/step -> {sb / elapsed * args.steps / 1e9:.1f} GB/s end to end (rounds "
          f"{gpu_rounds})", file=sys.stderr, flush=True)

    # per-step times: an event between consecutive replays (a separate pass)
    cur = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for _ in range(3):
        run()
    evs[0].record(cur)
    for i in range(args.steps):
        run()
        evs[i + 1].record(cur)
    torch.cuda.synchronize()
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    step_stats = {"median": round(float(np.median(step_ms)), 5), "min": round(float(step_ms.min()), 5),
                  "max": round(float(step_ms.max()), 5), "p10": round(float(np.percentile(step_ms, 10)), 5),
                  "p90": round(float(np.percentile(step_ms, 90)), 5),
                  "spread_pct": round(100 * float((np.percentile(step_ms, 90) - np.percentile(step_ms, 10))
                                                  / np.median(step_ms)), 2), "n": int(args.steps)}

    # profiled pass: events around every launch of every kind
    kinds = {Q.QD_K_EMBED: "embed", Q.QD_K_QKV: "qkv_gemv", Q.QD_K_QKV_POST: "qkv_post",
             Q.QD_K_ATTN: "attention", Q.QD_K_MERGE: "attn_merge", Q.QD_K_O: "o_proj_gemv",
             Q.QD_K_GATEUP: "gate_up_gemv", Q.QD_K_DOWN: "down_gemv", Q.QD_K_LMHEAD: "lm_head_gemv",
             Q.QD_K_ARGMAX: "argmax", Q.QD_K_OTHER: "other", Q.QD_K_STEP: "step_kernel"}
    mask = 0
    for k in kinds:
        mask |= 1 << k
    steps_prof = min(args.steps, max(1, 8000 // (shape.n_layers * 8 + 8)))
    Q.qd_profile_enable(mask)
    for _ in range(steps_prof):
        step()
    torch.cuda.synchronize()
    per_kind = {}
    for k, name in kinds.items():
        n, ms = Q.qd_profile_read(k)
        if n:
            per_kind[k] = (n, ms)
    Q.qd_profile_enable(0)
    # the cost of an event pair itself: pairs recorded back to back on the same
    # stream with nothing between them; subtracted from each launch's average
    cal = []
    for _ in range(200):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        e1.record(cur)
        cal.append((e0, e1))
    torch.cuda.synchronize()
    pair_us = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in cal]))
    bpl = _bytes_per_launch(shape, B, ctx)
    bpl[Q.QD_K_STEP] = sb
    # Each launch's net duration is its event interval less the cost of an event pair.
    # In the replayed graph the kernels run back to back, and the step time also holds
    # the dispatch of every launch; that remainder, shared equally over the launches,
    # is added to each net duration to give the launch's slot in the replayed step.
    net_us = {k: 1e3 * ms / n - pair_us for k, (n, ms) in per_kind.items()}
    launches_per_step = sum(n for n, _ in per_kind.values()) / steps_prof
    net_step_us = sum(net_us[k] * n / steps_prof for k, (n, _) in per_kind.items())
    share_us = max(0.0, (ms_per_step * 1e3 - net_step_us) / launches_per_step)
    print(f"[bench] event pair with nothing between: {pair_us:.2f} us (subtracted); dispatch share "
          f"{share_us:.2f} us per launch ({launches_per_step:.0f} launches, net kernel time "
          f"{net_step_us:.1f} of {1e3 * ms_per_step:.1f} us per step)", file=sys.stderr)
    for k, (n, ms) in sorted(per_kind.items(), key=lambda kv_: -net_us[kv_[0]] * kv_[1][0]):
        slot = net_us[k] + share_us
        gbs = (bpl[k] / (slot * 1e-6) / 1e9) if k in bpl else float("nan")
        tr = kind_duration(trace, kinds[k])[0] if trace else None
        print(f"[bench]   {kinds[k]:>14}: {n // steps_prof:3d}/step net {net_us[k]:8.2f} us, slot {slot:8.2f} us "
              f"{gbs:8.1f} GB/s" + (f", kernel trace {tr:8.2f} us" if tr else ""), file=sys.stderr)
    dom = max((k for k in per_kind if k in bpl), key=lambda k: net_us[k] * per_kind[k][0])
    slot_s = (net_us[dom] + share_us) * 1e-6
    tr_us, tr_calls = kind_duration(trace, kinds[dom]) if trace else (None, 0)
    avg_s = tr_us * 1e-6 if tr_us else slot_s
    achieved = bpl[dom] / avg_s / 1e9
    traffic, traffic_src = traffic_from_profiles(wl.name, kinds[dom])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kinds[dom], "bytes_per_launch": int(bpl[dom]),
                "avg_launch_us": round(avg_s * 1e6, 3),
                "duration_source": (f"rocprofv3 kernel trace of a child run ({tr_calls} launches): {trace_src}"
                                    if tr_us else f"events: {trace_src}"),
                "event_slot_us": round(slot_s * 1e6, 3), "net_launch_us": round(net_us[dom], 3),
                "dispatch_share_us": round(share_us, 3), "event_pair_us": round(pair_us, 3),
                "traffic_source": traffic_src}

    cpu = None
    if oracle is not None:
        cpu = oracle.record(oracle.single_thread(6.0))
    probe_end = hbm_probe(torch)

    rec = {"metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "int8w" if shape.w_dtype == "i8" else ("f32" if shape.w_dtype == "f32" else "bf16"),
           "data": "synthetic",
           "config": {"workload": wl.name, "batch": B, "past": int(ctx.max()) if wl.past else None,
                      "ctx_range": list(wl.ctx_range) if wl.ctx_range else None},
           "launch": "hip_graph" if graph else "eager", "weight_copies": rotate,
           "step_ms": step_stats, "gpu_rounds_tokens_per_s": gpu_rounds,
           "eager_tokens_per_s": round(B * args.steps / el_eager, 2),
           "hbm_gbs_end_to_end": round(sb * args.steps / elapsed / 1e9, 1),
           "hbm_frac_end_to_end": round(sb * args.steps / elapsed / 1e9 / HBM_PEAK_GBS, 4),
           "bytes_per_step": int(sb),
           "hbm_probe_gbs": {"start": probe_start, "end": probe_end, "what": "1 GiB device copy x3, read + write"},
           "gpu": torch.cuda.get_device_name(0), "machine": machine_info(),
           "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)
    append_log(args.log, {"time": time.strftime("%Y-%m-%dT%H:%M:%S%z"), "argv": sys.argv[1:], "record": rec,
                          "versions": versions_info(torch), "step_ms_samples": [round(float(v), 5) for v in step_ms]})


if __name__ == "__main__":
    main()
