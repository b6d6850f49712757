"""Benchmark: forward + backward of one tensor-parallel rank's share of the
Transformer block on one MI355X, through libmtb's C ABI.

One step = mtb_block_fwd + mtb_block_bwd (MTB_PHASE_ALL, every weight
gradient written) on resident synthetic bf16 inputs of the seq-2048 TP=8 rank
share (hidden 4096, 4 local heads x 128, ffn chunk 2048, batch 4, causal,
GELU). Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload seq2048|seq512|seq4096]
    python bench.py --calibrate-copy MIB

The default workload is the seq-2048 rank share (the metric's target
configuration); --workload seq512 times the seq-512 TP=4 share (hidden 1024,
4 heads x 64, ffn chunk 1024, batch 8) and seq4096 the SwiGLU/GQA share.

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
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "launches": 5, "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4}), flush=True)

WORKLOADS = {
    "seq2048": ("C4", "TP=8 rank share of a hidden-4096 block: 4 local heads x 128, ffn chunk 2048, "
                      "batch 4, seq 2048, causal, GELU", "one tp8 rank share"),
    "seq512": ("C2", "TP=4 rank share of a hidden-1024 block: 4 local heads x 64, ffn chunk 1024, "
                     "batch 8, seq 512, GELU", "one tp4 rank share"),
    "seq4096": ("C5", "TP=8 rank share of a hidden-4096 SwiGLU/GQA block: 4 q / 1 kv heads x 128, "
                      "ffn chunk 1792 (gate+up 3584), batch 2, seq 4096", "one tp8 rank share"),
}


def model_flops(cfg) -> float:
    """3 x forward matmul FLOPs; attention counts 4*d per visible (query, key)."""
    T, H, d = cfg.tokens, cfg.hidden, cfg.head_dim
    nq, nkv, F = cfg.q_heads, cfg.kv_heads, cfg.ffn
    Fu = 2 * F if cfg.act == "swiglu" else F
    pairs = cfg.seq * (cfg.seq + 1) // 2 if cfg.causal else cfg.seq * cfg.seq
    fwd = (2 * T * H * (nq + 2 * nkv) * d + 4 * d * pairs * cfg.batch * nq + 2 * T * nq * d * H
           + 2 * T * H * Fu + 2 * T * F * H)
    return 3.0 * fwd


def run_gpu(cfg, steps, warmup, trace_what=None):
    import torch

    from transformer_layer_ln_amd import inputs, mtb

    dev = torch.device("cuda")
    dt = torch.bfloat16
    a = inputs.activations(cfg)
    w = mtb.device_weights(inputs.shard_weights(cfg, 0), cfg.act, dt, dev)
    blk = mtb.BlockShard(mtb.cfg_from(cfg), w, dev)
    x = torch.as_tensor(a["x"]).to(dev, dt)
    dout = torch.full_like(x, 1.0 / x.numel())      # loss = mean(out)
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
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    traces = {}
    ctx = []
    for what in (trace_what or []):
        traces[what] = mtb.Trace(what, steps)
    # one trace can be armed at a time: time the step with the first, then
    # run extra armed passes for the others outside the timed region
    first = next(iter(traces.values()), None)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if first is not None:
        first.__enter__()
    t0.record(st)
    for _ in range(steps):
        step()
    t1.record(st)
    if first is not None:
        first.__exit__(None, None, None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    kern = {}
    for what, tr in traces.items():
        if tr is not first:
            with tr:
                for _ in range(steps):
                    step()
        kern[what] = tr.mean_ms()
    assert torch.isfinite(out.float()).all() and torch.isfinite(dx.float()).all()
    return ms, wall, kern


def cpu_baseline(cfg, budget_s=20.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same
    workload: the same rank share with batch 1 of 4 (one sequence of 2048
    tokens), forward + backward, repeated until ~budget_s of CPU time."""
    import numpy as np

    from oracle import block as ob
    from transformer_layer_ln_amd import inputs

    sample = cfg.with_(batch=1)
    a = inputs.activations(sample)
    w = inputs.shard_weights(sample, 0)
    kw = dict(q_heads=sample.q_heads, kv_heads=sample.kv_heads, head_dim=sample.head_dim,
              act=sample.act, causal=sample.causal)
    times = []
    t_start = time.perf_counter()
    while True:
        t = time.perf_counter()
        _, cache = ob.block_forward(a["x"], w, **kw)
        ob.block_backward(a["g"], cache)
        times.append(time.perf_counter() - t)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    sec = float(np.median(times))
    threads = os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS")
    cores = int(threads) if threads else os.cpu_count()
    return {"value": model_flops(sample) / sec / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "ms_per_step": sec * 1e3,
            "sample": (f"fp64 NumPy oracle fwd+bwd of the same rank share at batch 1 of "
                       f"{cfg.batch} (seq {cfg.seq}, {sample.tokens} tokens), median of "
                       f"{len(times)} step(s)")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--workload", default="seq2048", choices=sorted(WORKLOADS))
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported "
              "(the other tensor-parallel ranks run the same kernels on their own GPUs)",
              file=sys.stderr)
        sys.exit(2)

    from transformer_layer_ln_amd import inputs, mtb

    key, desc, par = WORKLOADS[args.workload]
    cfg = inputs.CONFIGS[key]
    flops = model_flops(cfg)
    ms, wall, kern = run_gpu(cfg, args.steps, args.warmup,
                             trace_what=[mtb.TRACE_FC1_FWD, mtb.TRACE_LN1_FWD, mtb.TRACE_ATTN_FWD])
    tflops = flops / (ms * 1e-3) / 1e12

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

    res = {
        "metric": f"block fwd+bwd TFLOP/s (one TP-rank shard, bf16) at seq {cfg.seq}",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) x, N(0,1/fan_in) weights, dout = 1/numel",
        "config": {"workload": desc, "batch": cfg.batch, "seq_len": cfg.seq,
                   "hidden": cfg.hidden, "local_q_heads": cfg.q_heads,
                   "local_kv_heads": cfg.kv_heads, "head_dim": cfg.head_dim,
                   "ffn_chunk": cfg.ffn, "parallelism": par},
        "model_flops_per_step": flops,
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(cfg.tokens / (ms * 1e-3), 1),
        "roofline": {"kernel": f"fc1 forward GEMM + {cfg.act} epilogue ({T} x {Fu} x {H})",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload), "traffic_unit": "bytes/launch",
                     "algorithmic_flops_per_launch": fc1_flops, "avg_ms": round(fc1_ms, 5)},
        "other_kernels": {
            "ln1_fwd": {"bound": "hbm", "avg_ms": round(ln_ms, 5),
                        "achieved_GBs": round(ln_bytes / (ln_ms * 1e-3) / 1e9, 1),
                        "peak_GBs": PEAK_HBM_GBS},
            "attn_fwd": {"bound": "mfma", "avg_ms": round(attn_ms, 5),
                         "achieved_TFLOPs": round(attn_flops / (attn_ms * 1e-3) / 1e12, 1)},
        },
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
