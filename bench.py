"""Benchmark: forward + backward of one tensor-parallel rank's share of the
Transformer block on one MI355X, through libmtb's C ABI.

One step = mtb_block_fwd + mtb_block_bwd (MTB_PHASE_ALL, every weight
gradient written) on resident synthetic bf16 inputs of the seq-2048 TP=8 rank
share (hidden 4096, 4 local heads x 128, ffn chunk 2048, batch 4, causal,
GELU), with a seeded N(0,1) upstream gradient. Prints ONE JSON line, which
also carries the metric's seq-512 leg (the seq-512 TP=4 share) and the same
step timed with the listing's loss mean(out).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload seq2048|seq512|seq4096|seq4096-causal|seq2048-post|seq2048-dropout]
    python bench.py --calibrate-copy MIB
    python bench.py --sweep

The default workload is the seq-2048 rank share (the metric's target
configuration); --workload seq512 times the seq-512 TP=4 share (hidden 1024,
4 heads x 64, ffn chunk 1024, batch 8) and seq4096 the SwiGLU/GQA share.

Besides the headline step it reports per-step median/p10/p90, the pages'
attention / FFN / backward segment times (library segment events), LN
forward/backward and attention-forward kernel rates, and, against HBM
bandwidth, the vocab-parallel cross-entropy (partial + loss + gradient) on
one [8192 x 16032] vocab shard and the vocab-parallel input embedding
(forward lookup, backward scatter-add) on one [16032 x 4096] table shard.

--sweep times the seq-512 share at seq 128/256/512/1024 and fits the
log-log slopes of the attention / FFN / backward times against seq.

--calibrate-copy runs only a plain device-to-device copy of MIB MiB, five
times, so that rocprofv3's FETCH_SIZE / WRITE_SIZE counters can be scaled
against a kernel whose HBM traffic is known (MIB MiB read + MIB MiB written
per launch).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# HBM bytes per fc1 launch from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE)
# scaled by the same counters on a copy of known size; valid only while the
# GEMM source is the one the counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_gemm_gelu_seq2048_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "transformer_layer_ln_amd", "csrc", f)
                for f in ("gemm.hip", "common.h", "kernels.h")]


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """traffic_bytes_per_launch from the committed counter summary, or None
    when there is none for this workload or the GEMM source has changed."""
    if workload != "seq2048" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != gemm_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    e0.record(st)
    for _ in range(4):
        dst.copy_(src)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 4
    print(json.dumps({"copy_mib": mib, "launches": 5, "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4, "avg_ms": round(ms, 4),
                      "GBs_read_plus_write": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)

WORKLOADS = {
    "seq2048": ("C4", "TP=8 rank share of a hidden-4096 block: 4 local heads x 128, ffn chunk 2048, "
                      "batch 4, seq 2048, causal, GELU", "one tp8 rank share"),
    "seq512": ("C2", "TP=4 rank share of a hidden-1024 block: 4 local heads x 64, ffn chunk 1024, "
                     "batch 8, seq 512, GELU", "one tp4 rank share"),
    "seq4096": ("C5", "TP=8 rank share of a hidden-4096 SwiGLU/GQA block: 4 q / 1 kv heads x 128, "
                      "ffn chunk 1792 (gate+up 3584), batch 2, seq 4096", "one tp8 rank share"),
    "seq4096-causal": ("C5c", "TP=8 rank share of a hidden-4096 SwiGLU/GQA block: 4 q / 1 kv heads x "
                              "128, ffn chunk 1792 (gate+up 3584), batch 2, seq 4096, causal",
                       "one tp8 rank share"),
    "seq2048-dropout": ("C4d", "TP=8 rank share of a hidden-4096 block: 4 local heads x 128, ffn chunk "
                               "2048, batch 4, seq 2048, causal, GELU, dropout 0.1 on the attention "
                               "probabilities and on the hidden state (counter-based masks)",
                        "one tp8 rank share"),
    "seq2048-post": ("C4p", "TP=8 rank share of a hidden-4096 block in post-LN order: 4 local heads "
                            "x 128, ffn chunk 2048, batch 4, seq 2048, causal, GELU",
                     "one tp8 rank share"),
}


def workload_cfg(key):
    from transformer_layer_ln_amd import inputs

    if key == "C5c":
        return inputs.C5.with_(name="C5-tp8-s4096-swiglu-gqa-causal", causal=True)
    if key == "C4p":
        return inputs.C4.with_(name="C4-tp8-s2048-post-ln", norm="post")
    if key == "C4d":
        return inputs.C4.with_(name="C4-tp8-s2048-dropout", p_attn=0.1, p_hidden=0.1,
                               drop_seed=1234, drop_offset=0)
    return inputs.CONFIGS[key]


def seq_sweep(steps, warmup):
    """The seq-512 TP=4 share at seq 128/256/512/1024 (batch 8): the pages'
    attention / FFN / backward segments per seq, and their log-log slopes
    against seq (attention kernel ~ s^2, FFN ~ s)."""
    import numpy as np

    from transformer_layer_ln_amd import inputs, mtb

    pts = []
    for sq in inputs.C3_SEQS:
        cfg = inputs.C3(sq)
        ms_e, _, _, kern, graph = run_gpu(cfg, steps, warmup,
                                          trace_what=[mtb.TRACE_ATTN_FWD, mtb.TRACE_ATTN_SEG,
                                                      mtb.TRACE_FFN_SEG, mtb.TRACE_BWD],
                                          graph_steps=steps)
        ms = graph[0]
        pts.append({"seq": sq, "tokens": cfg.tokens, "ms_per_step": round(ms, 4),
                    "ms_per_step_eager": round(ms_e, 4),
                    "attention_kernel_ms": round(kern[mtb.TRACE_ATTN_FWD], 5),
                    "attention_segment_ms": round(kern[mtb.TRACE_ATTN_SEG], 5),
                    "ffn_segment_ms": round(kern[mtb.TRACE_FFN_SEG], 5),
                    "backward_ms": round(kern[mtb.TRACE_BWD], 5),
                    "TFLOPs": round(model_flops(cfg) / (ms * 1e-3) / 1e12, 2)})
    ls = np.log([p["seq"] for p in pts])
    slope = lambda k: round(float(np.polyfit(ls, np.log([p[k] for p in pts]), 1)[0]), 3)
    return {"sweep": "seq", "workload": ("TP=4 rank share of a hidden-1024 block: 4 local heads x 64, "
                                         "ffn chunk 1024, batch 8, GELU, seq 128/256/512/1024"),
            "steps": steps, "warmup": warmup, "points": pts,
            "loglog_slope_vs_seq": {k: slope(k) for k in ("attention_kernel_ms", "attention_segment_ms",
                                                           "ffn_segment_ms", "backward_ms")}}


def model_flops(cfg) -> float:
    """3 x forward matmul FLOPs; attention counts 4*d per visible (query, key)."""
    T, H, d = cfg.tokens, cfg.hidden, cfg.head_dim
    nq, nkv, F = cfg.q_heads, cfg.kv_heads, cfg.ffn
    Fu = 2 * F if cfg.act == "swiglu" else F
    pairs = cfg.seq * (cfg.seq + 1) // 2 if cfg.causal else cfg.seq * cfg.seq
    fwd = (2 * T * H * (nq + 2 * nkv) * d + 4 * d * pairs * cfg.batch * nq + 2 * T * nq * d * H
           + 2 * T * H * Fu + 2 * T * F * H)
    return 3.0 * fwd


def run_gpu(cfg, steps, warmup, trace_what=None, graph_steps=0, cotangent="normal"):
    """Times `steps` fwd+bwd steps (one event pair around the whole timed
    region and one per step); returns (mean ms, per-step ms list, wall s,
    {trace: mean ms}, graph) with graph = (mean ms, per-step ms) of
    `graph_steps` replays of the step captured in a HIP graph, or None. The
    first trace is armed during the timed eager steps, the others during
    extra passes. cotangent: "normal" = the seeded N(0,1) upstream gradient
    the parity tests use (the headline: varied data, as in training);
    "mean" = the listing's loss mean(out), dout = 1/numel everywhere (a
    constant operand runs some GEMMs faster than varied data)."""
    import torch

    from transformer_layer_ln_amd import inputs, mtb

    dev = torch.device("cuda")
    dt = torch.bfloat16
    a = inputs.activations(cfg)
    w = mtb.device_weights(inputs.shard_weights(cfg, 0), cfg.act, dt, dev)
    blk = mtb.BlockShard(mtb.cfg_from(cfg), w, dev)
    x = torch.as_tensor(a["x"]).to(dev, dt)
    if cotangent == "mean":
        dout = torch.full_like(x, 1.0 / x.numel())  # loss = mean(out)
    else:
        dout = torch.as_tensor(a["g"]).to(dev, dt)  # seeded N(0,1) cotangent
    out = torch.empty_like(x)
    dx = torch.empty_like(x)
    grads = blk.grad_buffers()

    def step():
        blk.fwd(x, out)
        blk.bwd(x, dout, dx, grads)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    traces = {what: mtb.Trace(what, steps) for what in (trace_what or [])}
    first = next(iter(traces.values()), None)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if first is not None:
        first.__enter__()
    ev[0].record(st)
    for i in range(steps):
        step()
        ev[i + 1].record(st)
    if first is not None:
        first.__exit__(None, None, None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev[0].elapsed_time(ev[steps]) / steps
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    kern = {}
    for what, tr in traces.items():
        if tr is not first:
            with tr:
                for _ in range(steps):
                    step()
        kern[what] = tr.mean_ms()
    assert torch.isfinite(out.float()).all() and torch.isfinite(dx.float()).all()
    graph = None
    if graph_steps:
        # the same step captured once in a HIP graph and replayed: the kernels
        # and buffers are identical, only the per-launch host work is gone
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(graph_steps + 1)]
        torch.cuda.synchronize()
        gev[0].record(st)
        for i in range(graph_steps):
            g.replay()
            gev[i + 1].record(st)
        torch.cuda.synchronize()
        graph = (gev[0].elapsed_time(gev[graph_steps]) / graph_steps,
                 [gev[i].elapsed_time(gev[i + 1]) for i in range(graph_steps)])
        assert torch.isfinite(out.float()).all() and torch.isfinite(dx.float()).all()
    return ms, per_step, wall, kern, graph


def run_embed(ecfg, steps, warmup):
    """Vocab-parallel embedding forward and backward on vocab shard 0.
    Returns (fwd ms, bwd ms, tokens whose id lies in the shard)."""
    import torch

    from transformer_layer_ln_amd import inputs, mtb

    dev = torch.device("cuda")
    n, h, vl = ecfg.n_tokens, ecfg.hidden, ecfg.v_local
    ids_h = inputs.embed_ids(ecfg)
    ids = torch.as_tensor(ids_h).to(dev)
    table = torch.as_tensor(inputs.embed_table(ecfg, 0)).to(dev, torch.bfloat16)
    dout = torch.as_tensor(inputs.embed_dout(ecfg)).to(dev, torch.bfloat16)
    out = torch.empty(n, h, dtype=torch.bfloat16, device=dev)
    dtab = torch.empty_like(table)
    ws = torch.empty(mtb.vocab_embed_bwd_workspace_bytes(n, vl), dtype=torch.uint8, device=dev)
    fwd = lambda: mtb.vocab_embed_fwd(n, vl, 0, h, mtb.BF16, ids, table, out)
    bwd = lambda: mtb.vocab_embed_bwd(n, vl, 0, h, mtb.BF16, ids, dout, dtab, ws)
    st = torch.cuda.current_stream()
    res = []
    for call in (fwd, bwd):
        for _ in range(warmup):
            call()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(steps):
            call()
        e1.record(st)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / steps)
    own = int(((ids_h >= 0) & (ids_h < vl)).sum())
    return res[0], res[1], own


def run_lmhead(lcfg, steps, warmup):
    """Fused LM head + cross-entropy on the last vocab shard, no reduction
    hook (the shard's statistics are final). Returns (fwd ms, bwd ms) with
    the logits never stored, then (fwd ms, bwd ms) with the logits kept by
    the forward for the backward."""
    import torch

    from transformer_layer_ln_amd import inputs, mtb

    dev = torch.device("cuda")
    n, H, vl = lcfg.n_tokens, lcfg.hidden, lcfg.v_local
    v0 = (lcfg.tp - 1) * vl
    h = torch.as_tensor(inputs.lmhead_h(lcfg)).to(dev, torch.bfloat16)
    w = torch.as_tensor(inputs.lmhead_w(lcfg, lcfg.tp - 1)).to(dev, torch.bfloat16)
    t = torch.as_tensor(v0 + inputs.lmhead_targets(lcfg) % vl).to(dev)
    dl = torch.full((n,), 1.0 / n, dtype=torch.float32, device=dev)
    stats = torch.empty(4, n, dtype=torch.float32, device=dev)
    loss = torch.empty(n, dtype=torch.float32, device=dev)
    dh = torch.empty_like(h)
    dw = torch.empty_like(w)
    ws = torch.empty(mtb.lmhead_xent_workspace_bytes(n, H, vl), dtype=torch.uint8, device=dev)
    z = torch.empty(n, vl, dtype=torch.bfloat16, device=dev)
    fwd = lambda: mtb.lmhead_xent_fwd(n, H, vl, v0, mtb.BF16, h, w, t, stats, loss, ws)
    bwd = lambda: mtb.lmhead_xent_bwd(n, H, vl, v0, mtb.BF16, h, w, t, stats, dl, dh, dw, ws)
    fwd_s = lambda: mtb.lmhead_xent_fwd(n, H, vl, v0, mtb.BF16, h, w, t, stats, loss, ws, logits=z)

    def bwd_s():   # the backward overwrites the stored logits with dz: store them again first
        fwd_s()
        mtb.lmhead_xent_bwd(n, H, vl, v0, mtb.BF16, h, w, t, stats, dl, dh, dw, None, logits=z)

    st = torch.cuda.current_stream()
    res = []
    for call in (fwd, bwd, fwd_s, bwd_s):
        for _ in range(warmup):
            call()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(steps):
            call()
        e1.record(st)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / steps)
    return res[0], res[1], res[2], res[3] - res[2]


def run_xent(xcfg, steps, warmup):
    """X1-X3 on one vocab shard: mtb_vocab_xent(MTB_XENT_ALL) with the
    identity reduction (one shard's statistics are final), loss and the
    logit gradient into a separate buffer. Returns mean ms per call."""
    import torch

    from transformer_layer_ln_amd import inputs, mtb

    dev = torch.device("cuda")
    n, v = xcfg.n_tokens, xcfg.v_local
    z = torch.as_tensor(inputs.xent_logits(xcfg, 0)).to(dev, torch.bfloat16)
    y = torch.as_tensor(inputs.xent_targets(xcfg)).to(dev)
    dl = torch.as_tensor(inputs.xent_dloss(xcfg)).to(dev)
    stats = torch.empty(4 * n, dtype=torch.float32, device=dev)
    loss = torch.empty(n, dtype=torch.float32, device=dev)
    dz = torch.empty_like(z)

    def call():
        mtb.vocab_xent(n, v, 0, mtb.BF16, mtb.XENT_ALL, z, y, stats, loss, dl, dz)

    for _ in range(warmup):
        call()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    assert torch.isfinite(loss).all()
    return e0.elapsed_time(e1) / steps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """The host threads this process may use: its CPU affinity, capped by a
    thread-count limit the environment sets (the GPU machine's per-GPU share)."""
    n = len(os.sched_getaffinity(0))
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit() and int(v) > 0:
            n = min(n, int(v))
    return max(1, n)


def cpu_child(key, budget_s):
    """Runs in a child process (its BLAS thread count fixed by the parent's
    environment). Waits for one line on stdin, then times the fp64 oracle
    (as it stands) on a bounded sample of the workload -- the same rank share
    at batch 1 (one sequence), forward + backward, median of up to 3 steps
    within ~budget_s -- and prints one JSON line."""
    import numpy as np

    sys.stdin.readline()
    from oracle import block as ob
    from transformer_layer_ln_amd import inputs

    cfg = workload_cfg(key)
    sample = cfg.with_(batch=1)
    a = inputs.activations(sample)
    w = inputs.shard_weights(sample, 0)
    kw = dict(q_heads=sample.q_heads, kv_heads=sample.kv_heads, head_dim=sample.head_dim,
              act=sample.act, causal=sample.causal, norm=sample.norm)
    if sample.p_attn or sample.p_hidden:
        kw["dropout"] = dict(p_attn=sample.p_attn, p_hidden=sample.p_hidden,
                             seed=sample.drop_seed, offset=sample.drop_offset)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        # numpy's (and scipy's, if loaded) BLAS, each limited by the environment
        threads = max(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        pass
    times = []
    t_start = time.perf_counter()
    while True:
        t = time.perf_counter()
        _, cache = ob.block_forward(a["x"], w, **kw)
        ob.block_backward(a["g"], cache)
        times.append(time.perf_counter() - t)
        if time.perf_counter() - t_start > budget_s or len(times) >= 3:
            break
    sec = float(np.median(times))
    print(json.dumps({"sec": sec, "steps": len(times), "blas_threads": threads,
                      "flops": model_flops(sample), "tokens": sample.tokens}), flush=True)


def start_cpu_children(key, budget_s):
    """The oracle's timing processes, started before this process makes any
    GPU call (they compute only when told to, after the GPU timings): one at
    the threads this process may use, one at a single thread."""
    import subprocess

    kids = []
    for n in sorted({cpu_threads(), 1}, reverse=True):
        env = dict(os.environ, OPENBLAS_NUM_THREADS=str(n), OMP_NUM_THREADS=str(n),
                   MKL_NUM_THREADS=str(n))
        p = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-child", key,
                              "--cpu-budget", str(budget_s)],
                             stdin=subprocess.PIPE, stdout=subprocess.PIPE, env=env, text=True)
        kids.append((n, p))
    return kids


def finish_cpu_children(kids, cfg):
    """Runs the children one after the other and folds their timings into
    the cpu_baseline object (the all-thread run is the reported value)."""
    runs = []
    for n, p in kids:
        out, _ = p.communicate("go\n", timeout=600)
        if p.returncode != 0:
            raise RuntimeError(f"oracle timing child ({n} threads) failed: {p.returncode}")
        r = json.loads(out.strip().splitlines()[-1])
        runs.append({"threads": n, "blas_threads": r["blas_threads"],
                     "ms_per_step": round(r["sec"] * 1e3, 1), "steps": r["steps"],
                     "value": r["flops"] / r["sec"] / 1e12})
    best = runs[0]
    return {"value": best["value"], "unit": "TFLOP/s", "cores": best["threads"], "kind": "oracle",
            "ms_per_step": best["ms_per_step"],
            "sample": (f"fp64 NumPy oracle fwd+bwd of the same rank share at batch 1 of "
                       f"{cfg.batch} (seq {cfg.seq}, {cfg.seq} tokens), median of up to 3 steps "
                       "in a child process started before any GPU call"),
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "runs": runs}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--workload", default="seq2048", choices=sorted(WORKLOADS))
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--sweep", action="store_true", help="seq 128..1024 sweep of the seq-512 share")
    ap.add_argument("--eager", action="store_true", help="time eager library calls, not graph replays")
    ap.add_argument("--cpu-child", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_child:
        cpu_child(args.cpu_child, args.cpu_budget)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported "
              "(the other tensor-parallel ranks run the same kernels on their own GPUs)",
              file=sys.stderr)
        sys.exit(2)

    from transformer_layer_ln_amd import inputs, mtb

    if args.sweep:
        print(json.dumps(seq_sweep(args.steps, args.warmup)), flush=True)
        return
    key, desc, par = WORKLOADS[args.workload]
    kids = [] if args.no_cpu_baseline else start_cpu_children(key, args.cpu_budget)
    cfg = workload_cfg(key)
    flops = model_flops(cfg)
    ms_eager, per_step_eager, wall, kern, graph = run_gpu(
        cfg, args.steps, args.warmup,
        trace_what=[mtb.TRACE_FC1_FWD, mtb.TRACE_LN1_FWD, mtb.TRACE_ATTN_FWD, mtb.TRACE_ATTN_SEG,
                    mtb.TRACE_FFN_SEG, mtb.TRACE_BWD, mtb.TRACE_LN1_BWD, mtb.TRACE_FC2_WGRAD],
        graph_steps=0 if args.eager else args.steps)
    ms, per_step = (ms_eager, per_step_eager) if graph is None else graph
    tflops = flops / (ms * 1e-3) / 1e12
    # the same step with the listing's loss, mean(out): dout = 1/numel everywhere
    ms_m_eager, _, _, _, graph_m = run_gpu(cfg, args.steps, args.warmup,
                                           graph_steps=0 if args.eager else args.steps,
                                           cotangent="mean")
    ms_mean = ms_m_eager if graph_m is None else graph_m[0]
    # the metric's seq-512 leg: the seq-512 TP=4 rank share, same timing
    legs = {}
    if args.workload == "seq2048":
        c2 = workload_cfg("C2")
        e2, _, _, _, g2 = run_gpu(c2, args.steps, args.warmup,
                                  graph_steps=0 if args.eager else args.steps)
        ms2 = e2 if g2 is None else g2[0]
        f2 = model_flops(c2)
        legs["seq512"] = {"workload": WORKLOADS["seq512"][1], "ms_per_step": round(ms2, 4),
                          "TFLOPs": round(f2 / (ms2 * 1e-3) / 1e12, 2),
                          "frac_of_bf16_peak": round(f2 / (ms2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "model_flops_per_step": f2}
    srt = sorted(per_step)
    pct = lambda q: srt[min(len(srt) - 1, int(q * (len(srt) - 1) + 0.5))]

    T, H, F = cfg.tokens, cfg.hidden, cfg.ffn
    Fu = 2 * F if cfg.act == "swiglu" else F
    fc1_flops = 2.0 * T * H * Fu
    fc1_ms = kern[mtb.TRACE_FC1_FWD]
    achieved = fc1_flops / (fc1_ms * 1e-3) / 1e12
    ln_bytes = T * H * 2 * 2 + T * 8          # read x, write a (bf16), write mu/rstd
    ln_ms = kern[mtb.TRACE_LN1_FWD]
    attn_pairs = cfg.seq * (cfg.seq + 1) // 2 if cfg.causal else cfg.seq * cfg.seq
    attn_flops = 4.0 * cfg.head_dim * attn_pairs * cfg.batch * cfg.q_heads
    attn_ms = kern[mtb.TRACE_ATTN_FWD]
    lnb_bytes = T * H * 2 * 4 + T * 8          # read dy, x, dres, write dx (bf16), read mu/rstd
    lnb_ms = kern[mtb.TRACE_LN1_BWD]
    # the fc2 and fc1 weight gradients, traced together (one grouped launch where
    # their tiles fill the chip together, else one launch each)
    wg_flops = 2.0 * T * H * F + 2.0 * T * Fu * H
    wg_ms = kern[mtb.TRACE_FC2_WGRAD]
    xcfg = inputs.C5_XENT
    xent_ms = run_xent(xcfg, args.steps, args.warmup)
    xent_bytes = 6 * xcfg.n_tokens * xcfg.v_local   # X1 reads 2 B/logit, X3 reads 2 + writes 2
    ecfg = inputs.C5_EMBED
    emb_f_ms, emb_b_ms, emb_own = run_embed(ecfg, args.steps, args.warmup)
    # forward: read the in-shard rows, write every output row; backward: read
    # the in-shard tokens' gradient rows, write every table row (+ 8 B ids)
    emb_f_bytes = (emb_own + ecfg.n_tokens) * ecfg.hidden * 2 + 8 * ecfg.n_tokens
    emb_b_bytes = (emb_own + ecfg.v_local) * ecfg.hidden * 2 + 8 * ecfg.n_tokens
    lcfg = inputs.C5_LMHEAD
    lm_f_ms, lm_b_ms, lm_fs_ms, lm_bs_ms = run_lmhead(lcfg, args.steps, args.warmup)
    lm_flops = 2.0 * lcfg.n_tokens * lcfg.hidden * lcfg.v_local   # one [n x V_r x H] product

    metric = ("block fwd+bwd TFLOP/s & ms/step (one TP-rank shard, bf16) at seq 512/2048"
              if args.workload == "seq2048" else
              f"block fwd+bwd TFLOP/s & ms/step (one TP-rank shard, bf16) at seq {cfg.seq}")
    res = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(pct(0.5), 4),
        "ms_per_step_p10": round(pct(0.1), 4),
        "ms_per_step_p90": round(pct(0.9), 4),
        "launch": ("eager: one library call per fwd and per bwd" if graph is None else
                   "HIP graph: one fwd+bwd step captured once, replayed per step"),
        "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) x, N(0,1/fan_in) weights, seeded N(0,1) upstream gradient",
        "ms_per_step_mean_loss": round(ms_mean, 4),
        "TFLOPs_mean_loss": round(flops / (ms_mean * 1e-3) / 1e12, 2),
        "mean_loss_note": ("the same step with the listing's loss mean(out), i.e. dout = 1/numel "
                           "everywhere: the constant operand runs the fc2 backward GEMMs faster"),
        "config": {"workload": desc, "batch": cfg.batch, "seq_len": cfg.seq,
                   "hidden": cfg.hidden, "local_q_heads": cfg.q_heads,
                   "local_kv_heads": cfg.kv_heads, "head_dim": cfg.head_dim,
                   "ffn_chunk": cfg.ffn, "parallelism": par},
        "model_flops_per_step": flops,
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(cfg.tokens / (ms * 1e-3), 1),
        "legs": legs,
        "roofline": {"kernel": f"fc1 forward GEMM + {cfg.act} epilogue ({T} x {Fu} x {H})",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload), "traffic_unit": "bytes/launch",
                     "algorithmic_flops_per_launch": fc1_flops, "avg_ms": round(fc1_ms, 5)},
        "other_kernels": {
            # the input LayerNorm's kernels (pre-LN order only: post-LN has none)
            "ln1_fwd": None if cfg.norm == "post" else {
                "bound": "hbm", "avg_ms": round(ln_ms, 5),
                "achieved_GBs": round(ln_bytes / (ln_ms * 1e-3) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS},
            "attn_fwd": {"bound": "mfma", "avg_ms": round(attn_ms, 5),
                         "achieved_TFLOPs": round(attn_flops / (attn_ms * 1e-3) / 1e12, 1)},
            "mlp_wgrad": {"bound": "mfma",
                          "what": ("fc2 and fc1 weight gradients (the step's longest launch when they "
                                   "run as one grouped launch)"),
                          "avg_ms": round(wg_ms, 5),
                          "achieved_TFLOPs": round(wg_flops / (wg_ms * 1e-3) / 1e12, 1),
                          "peak_TFLOPs": PEAK_BF16_TFLOPS},
            "ln1_bwd": None if cfg.norm == "post" else {
                "bound": "hbm", "avg_ms": round(lnb_ms, 5),
                "achieved_GBs": round(lnb_bytes / (lnb_ms * 1e-3) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS},
            "vocab_xent": {"bound": "hbm", "workload": (
                               f"one vocab shard [{xcfg.n_tokens} x {xcfg.v_local}] bf16 of "
                               f"V={xcfg.vocab} over TP={xcfg.tp}: partial (max, sum exp, target "
                               "logit) + loss + logit gradient, identity reduction"),
                           "avg_ms": round(xent_ms, 5),
                           "achieved_GBs": round(xent_bytes / (xent_ms * 1e-3) / 1e9, 1),
                           "peak_GBs": PEAK_HBM_GBS},
            "vocab_embed": {"bound": "hbm", "workload": (
                                f"one vocab shard [{ecfg.v_local} x {ecfg.hidden}] bf16 of "
                                f"V={ecfg.vocab} over TP={ecfg.tp}, {ecfg.n_tokens} token ids "
                                f"({emb_own} in the shard)"),
                            "fwd_avg_ms": round(emb_f_ms, 5),
                            "fwd_achieved_GBs": round(emb_f_bytes / (emb_f_ms * 1e-3) / 1e9, 1),
                            "bwd_avg_ms": round(emb_b_ms, 5),
                            "bwd_achieved_GBs": round(emb_b_bytes / (emb_b_ms * 1e-3) / 1e9, 1),
                            "peak_GBs": PEAK_HBM_GBS},
            "lmhead_xent": {"bound": "mfma", "workload": (
                                f"LM head + cross-entropy on one vocab shard: [{lcfg.n_tokens} x "
                                f"{lcfg.hidden}] x [{lcfg.v_local} x {lcfg.hidden}]^T bf16 of "
                                f"V={lcfg.vocab} over TP={lcfg.tp}; forward = logits GEMM with "
                                "the loss statistics in its epilogue; backward = logits "
                                "recomputed with the gradient epilogue, then dh and dW GEMMs"),
                            "fwd_avg_ms": round(lm_f_ms, 5),
                            "fwd_achieved_TFLOPs": round(lm_flops / (lm_f_ms * 1e-3) / 1e12, 1),
                            "bwd_avg_ms": round(lm_b_ms, 5),
                            "bwd_achieved_TFLOPs": round(3 * lm_flops / (lm_b_ms * 1e-3) / 1e12,
                                                         1),
                            "stored_logits": {
                                "note": "logits kept by the forward (bf16, 263 MB) and used by the "
                                        "backward instead of recomputing them",
                                "fwd_avg_ms": round(lm_fs_ms, 5), "bwd_avg_ms": round(lm_bs_ms, 5),
                                "bwd_achieved_TFLOPs": round(2 * lm_flops / (lm_bs_ms * 1e-3) / 1e12,
                                                             1)},
                            "peak_TFLOPs": PEAK_BF16_TFLOPS},
        },
        # the pages' breakdown (attention / FFN / backward), timed by the
        # library's segment events; the pages' own figures are context only
        "segments_ms": {"attention_fwd": round(kern[mtb.TRACE_ATTN_SEG], 4),
                        "ffn_fwd": round(kern[mtb.TRACE_FFN_SEG], 4),
                        "backward": round(kern[mtb.TRACE_BWD], 4)},
        "context_pages": ("seq 512 on 4 unspecified GPUs, PyTorch eager: attention 18.42 ms, "
                          "FFN 21.76 ms, backward 40.35 ms per step"),
        "wall_s_timed": round(wall, 3),
    }
    if kids:
        res["cpu_baseline"] = finish_cpu_children(kids, cfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
