"""Decode-step benchmark on one MI355X: tokens/s and achieved HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one qd_decode_step call (timed as a HIP-graph replay of that call,
captured once; the eager-launch rate is reported beside it): embedding, every layer (fused RMSNorm + QKV
GEMV, q/k norm + RoPE + KV append, split-K attention + merge, o_proj + residual,
RMSNorm + gate/up + SwiGLU, down + residual), final norm, lm_head and greedy
argmax, for one batch of synthetic input already resident in HBM. Each step
re-runs the same positions (the step is idempotent at a position), so every
timed step attends over exactly `past` cached tokens.

Prints ONE JSON line. `roofline` covers the dominant kernel kind: its
algorithmic bytes per launch divided by its average launch duration, measured
with HIP events recorded on the library's stream around each launch of every
kind, in a second pass of the same steps right after the clean timed region
(net of an event pair's own cost, plus the launch's equal share of the
replayed step's dispatch time). `traffic` is the measured HBM bytes per launch
of that kernel from the hardware-counter summaries under profiles/, when they
were taken from the current sources.
`cpu_baseline` is the fp64 oracle timed on the host over a bounded sample of
whole decode steps of the same workload.
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
    return out


def step_bytes(shape, B, ctx):
    """Algorithmic bytes of one whole step (every weight once, every cached K/V once,
    the new K/V written, the embedding rows and the logits)."""
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


def cpu_baseline(wl, case_host, ctx, tokens, budget_s=12.0):
    """Whole oracle decode steps on the host until about budget_s seconds have
    run (at least two steps), after one untimed step that widens the weights."""
    from oracle.qwen2 import OracleWeights, decode_step
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    shape = wl.shape
    host_w, kh, vh, table = case_host
    ow = OracleWeights(shape, host_w, cache_layers=True)
    decode_step(shape, ow, kh, vh, table, ctx, tokens=tokens)
    n, t0 = 0, time.perf_counter()
    while True:
        decode_step(shape, ow, kh, vh, table, ctx, tokens=tokens)
        n += 1
        el = time.perf_counter() - t0
        if (el >= budget_s and n >= 2) or el > 4 * budget_s:
            break
    B = len(ctx)
    return {"value": round(B * n / el, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} whole decode steps of {wl.name} (batch {B}) in {el:.1f} s, fp64 numpy, "
                      f"after one untimed step that widens the weights"}


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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
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
           "attention_us": round(1e3 * ms_a / np_, 2), "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


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
        cpu = {"value": round(B * n / el, 2), "unit": "sampled tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} calls of the numpy oracle sampler over the same {B} x {V} logits in {el:.1f} s"}
    rec = {"metric": "sampled tokens/s, temperature/top-k/top-p sampler, 0.5B vocabulary",
           "value": round(B / (us * 1e-6), 1), "unit": "sampled tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": wl.name, "batch": B, "vocab": V, **X}, "launch": "eager",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "sample_kernel",
                        "bytes_per_launch": nbytes, "avg_launch_us": round(us, 3)},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen2-0.5b-bf16-b1-past512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device-to-device copy of 1 GiB (5 times): the reference kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU layout is described in DESIGN.md and not run.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_step_amd import qd as Q
    from decode_step_amd.runner import DecodeRunner
    from workloads import shapes as S, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        return copy_probe()
    wl = S.WORKLOADS[args.workload]
    if wl.kind == "prefill":
        return bench_prefill(wl, args)
    if wl.kind == "sample":
        return bench_sample(wl, args)
    shape = wl.shape
    dev = "cuda"
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
    runner = DecodeRunner(shape, w, kv.k, kv.v, kv.block_table, max_batch=B, max_ctx=int(ctx.max()) + 2,
                          device=dev)
    tokens = synth.make_tokens(B, shape.vocab, seed=wl.seed, name="tok0")
    tok_d = torch.from_numpy(tokens).to(dev)
    pos_d = torch.from_numpy(ctx).to(dev)
    logits = torch.empty(B, shape.vocab, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    def step():
        runner.step(ctx, pos_d, tokens=tok_d, logits=logits, next_tokens=nxt,
                    stream=torch.cuda.current_stream())

    def timed(fn, k):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    sb = step_bytes(shape, B, ctx)
    # eager launches (one qd_decode_step call per step)
    for _ in range(args.warmup):
        step()
    el_eager = timed(step, args.steps)
    print(f"[bench] {wl.name} eager: {1e3 * el_eager / args.steps:.4f} ms/step, "
          f"{B * args.steps / el_eager:.1f} tokens/s", file=sys.stderr, flush=True)
    # the same call captured once in a HIP graph and replayed (NEXT-2: one launch per step)
    graph = None
    if not args.no_graph:
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
        elapsed = timed(graph.replay, args.steps)
    else:
        elapsed = el_eager
    ms_per_step = 1e3 * elapsed / args.steps
    tok_s = B * args.steps / elapsed
    print(f"[bench] {wl.name} {'graph' if graph else 'eager'}: {ms_per_step:.4f} ms/step, {tok_s:.1f} tokens/s, "
          f"{sb / 1e6:.2f} MB/step -> {sb / elapsed * args.steps / 1e9:.1f} GB/s end to end",
          file=sys.stderr, flush=True)

    # profiled pass: events around every launch of every kind
    kinds = {Q.QD_K_EMBED: "embed", Q.QD_K_QKV: "qkv_gemv", Q.QD_K_QKV_POST: "qkv_post",
             Q.QD_K_ATTN: "attention", Q.QD_K_MERGE: "attn_merge", Q.QD_K_O: "o_proj_gemv",
             Q.QD_K_GATEUP: "gate_up_gemv", Q.QD_K_DOWN: "down_gemv", Q.QD_K_LMHEAD: "lm_head_gemv",
             Q.QD_K_ARGMAX: "argmax", Q.QD_K_OTHER: "other"}
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
    # (the rocprofv3 kernel duration has no such term)
    cal = []
    cur = torch.cuda.current_stream()
    for _ in range(200):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        e1.record(cur)
        cal.append((e0, e1))
    torch.cuda.synchronize()
    pair_us = float(np.mean([1e3 * a_.elapsed_time(b_) for a_, b_ in cal]))
    bpl = _bytes_per_launch(shape, B, ctx)
    # Each launch's net duration is its event interval less the cost of an event pair.
    # In the replayed graph the kernels run back to back, and the step time also holds
    # the dispatch of every launch; that remainder, shared equally over the launches,
    # is added to each net duration to give the launch's slot in the replayed step
    # (the slots sum to the step time; rocprofv3's kernel durations of a graph replay
    # tile the step the same way).
    net_us = {k: 1e3 * ms / n - pair_us for k, (n, ms) in per_kind.items()}
    launches_per_step = sum(n for n, _ in per_kind.values()) / steps_prof
    net_step_us = sum(net_us[k] * n / steps_prof for k, (n, _) in per_kind.items())
    share_us = max(0.0, (ms_per_step * 1e3 - net_step_us) / launches_per_step)
    total_ms = sum(ms for _, ms in per_kind.values())
    print(f"[bench] event pair with nothing between: {pair_us:.2f} us (subtracted); dispatch share "
          f"{share_us:.2f} us per launch ({launches_per_step:.0f} launches, net kernel time "
          f"{net_step_us:.1f} of {1e3 * ms_per_step:.1f} us per step)", file=sys.stderr)
    for k, (n, ms) in sorted(per_kind.items(), key=lambda kv_: -net_us[kv_[0]] * kv_[1][0]):
        slot = net_us[k] + share_us
        gbs = (bpl[k] / (slot * 1e-6) / 1e9) if k in bpl else float("nan")
        print(f"[bench]   {kinds[k]:>14}: {n // steps_prof:3d}/step net {net_us[k]:8.2f} us, slot {slot:8.2f} us "
              f"{gbs:8.1f} GB/s", file=sys.stderr)
    dom = max((k for k in per_kind if k in bpl), key=lambda k: net_us[k] * per_kind[k][0])
    n_dom = per_kind[dom][0]
    avg_s = (net_us[dom] + share_us) * 1e-6
    achieved = bpl[dom] / avg_s / 1e9
    traffic, traffic_src = traffic_from_profiles(wl.name, kinds[dom])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kinds[dom], "bytes_per_launch": int(bpl[dom]),
                "avg_launch_us": round(avg_s * 1e6, 3), "net_launch_us": round(net_us[dom], 3),
                "dispatch_share_us": round(share_us, 3), "event_pair_us": round(pair_us, 3),
                "traffic_source": traffic_src}

    cpu = None
    if not args.no_cpu_baseline:
        if shape.w_dtype == "i8":   # the oracle runs the same codes dequantized
            from oracle.quant import quantized_model
            hw = quantized_model(host_w)[0]
        else:
            hw = synth.weights_to_host(w)
        case_host = (hw, [synth.to_host_bits(t).copy() for t in kv.k],
                     [synth.to_host_bits(t).copy() for t in kv.v], kv.block_table)
        cpu = cpu_baseline(wl, case_host, ctx, tokens)

    rec = {"metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "int8w" if shape.w_dtype == "i8" else ("f32" if shape.w_dtype == "f32" else "bf16"),
           "data": "synthetic",
           "config": {"workload": wl.name, "batch": B, "past": int(ctx.max()) if wl.past else None,
                      "ctx_range": list(wl.ctx_range) if wl.ctx_range else None},
           "launch": "hip_graph" if graph else "eager",
           "eager_tokens_per_s": round(B * args.steps / el_eager, 2),
           "hbm_gbs_end_to_end": round(sb * args.steps / elapsed / 1e9, 1),
           "hbm_frac_end_to_end": round(sb * args.steps / elapsed / 1e9 / HBM_PEAK_GBS, 4),
           "bytes_per_step": int(sb),
           "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
