#!/usr/bin/env python3
"""Throughput of the sparse flash attention backward on one MI355X.

One step = one full backward call (index decode, Delta, accumulator fill, the
MFMA kernels, the dK/dV scatter or key-centric reduction, and the cast) over
one batch of synthetic inputs already resident in HBM.  The default workload
is the DSA-style training shape: BSND, B=1, S1=S2=4096, N1=128 heads sharing
one key/value head, D=512 plus a 64-wide rope part, K=2048 causal top-k
indices (25% local window, 75% uniform), bf16.

Prints one JSON line with the whole-job TFLOP/s (5504 flop per valid
(head, selected position) pair, 5120 without rope), the roofline of the
dominant kernel measured with HIP events inside the timed region, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def _count_valid(case, inp, sfag):
    """Valid (token, position) pairs and per-token counts via the library's index decode."""
    import torch
    idx = inp["sparse_indices"].reshape(case.T1, case.Kent)
    kw = dict(T2=case.T2, block_size=case.block, layout=case.layout, sparse_mode=case.mode)
    if case.layout == "TND":
        kw.update(seqlens_q=inp["seqlens_q"], seqlens_kv=inp["seqlens_kv"])
    else:
        kw.update(B=case.B, S1=case.S1, S2=case.S2)
    nv, rows, off, pairs = sfag.build_index(idx, **kw)
    torch.cuda.synchronize()
    n = int(nv.to(torch.int64).sum().item())
    del rows, off, pairs
    return n, nv


def _alg_bytes(case, n_pairs):
    """No-reuse algorithmic bytes of one backward call."""
    e = 2
    G, D, Dr, T1, T2 = case.G, case.D, case.Dr, case.T1, case.T2
    per_token = G * (D + Dr) * e * 2 + G * D * e * 2 + G * 4 * 2 + G * 4 * 2 + case.Kent * 4
    per_pair = (2 * D + Dr) * e + (2 * D + Dr) * 4
    per_key = (2 * D + Dr) * 4 * 2 + (2 * D + Dr) * e
    return T1 * per_token + n_pairs * per_pair + T2 * per_key


def _cpu_baseline(case, inp, seed, target_s=15.0):
    """The oracle as it stands, on one host thread, over a seeded sample of
    tokens: each sampled token's full backward (its dQ row and its dK/dV
    scatter).  Batches double in size until about ``target_s`` seconds."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import sfag_oracle as orc
    T1 = case.T1
    order = np.random.default_rng(seed).permutation(T1)
    cpu = lambda x, shape: None if x is None else x.detach().reshape(shape)
    G, D, Dr = case.G, case.D, case.Dr
    if case.layout == "BSND":
        geom = orc.geometry("BSND", case.B, case.S1, case.S2)
    else:
        geom = orc.geometry("TND", case.B, seqlens_q=case.seqlens_q, seqlens_kv=case.seqlens_kv)
    k = inp["key"].detach().reshape(case.T2, D).cpu()
    v = inp["value"].detach().reshape(case.T2, D).cpu()
    kr = inp["key_rope"].detach().reshape(case.T2, Dr).cpu() if Dr else None
    full = dict(q=cpu(inp["query"], (T1, G, D)), dO=cpu(inp["dout"], (T1, G, D)), O=cpu(inp["out"], (T1, G, D)),
                m=cpu(inp["softmax_max"], (T1, G)), l=cpu(inp["softmax_sum"], (T1, G)),
                qr=cpu(inp.get("query_rope"), (T1, G, Dr)) if Dr else None,
                idx=cpu(inp["sparse_indices"], (T1, case.Kent)))
    done, flops, used, batch = 0, 0, 0.0, 2
    with threadpool_limits(limits=1):
        while used < target_s and done < T1:
            sel = np.sort(order[done:done + batch])
            ts = __import__("torch").as_tensor(sel)
            sub = {n: None if x is None else x[ts.to(x.device)].cpu() for n, x in full.items()}
            g = {n: (a[sel] if isinstance(a, np.ndarray) else a) for n, a in geom.items()}
            g["T1"] = len(sel)
            t0 = time.perf_counter()
            orc.backward(sub["q"], k, v, sub["qr"], kr, sub["idx"], sub["dO"], sub["O"], sub["m"], sub["l"], g,
                         case.block, case.mode, case.scale_value)
            used += time.perf_counter() - t0
            flops += orc.flops(orc.decode(sub["idx"], case.block, case.mode, g), G, D, Dr)
            done += len(sel)
            batch *= 2
    return dict(value=flops / used / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                sample=f"{done} seeded tokens of the same workload, each token's full backward (dQ row and dK/dV "
                       f"scatter), float64 NumPy on one thread, {used:.1f} s")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2, help="workload number (1-5); 2 is the headline")
    ap.add_argument("--deterministic", choices=("config", "true", "false"), default="config")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures a single GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch

    import sfag_inputs as si
    import top_sparse_attention_sfag_amd as sfag

    case = si.CONFIGS[args.config]
    det = case.deterministic if args.deterministic == "config" else args.deterministic == "true"
    seed = si.seed_for(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {case.name} on {dev}", file=sys.stderr, flush=True)
    inp = si.make_inputs(case, seed, device=dev)
    inp.update(si.standin_stats(case, inp, seed, device=dev))
    torch.cuda.synchronize()
    n_pairs, _ = _count_valid(case, inp, sfag)
    flop_per_pair = 2 * (3 * (case.D + case.Dr) + 2 * case.D)
    flops = n_pairs * case.G * flop_per_pair

    outs = (torch.empty_like(inp["query"]), torch.empty_like(inp["key"]), torch.empty_like(inp["value"]),
            torch.empty_like(inp["query_rope"]) if case.Dr else None,
            torch.empty_like(inp["key_rope"]) if case.Dr else None)
    kw = dict(seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"), query_rope=inp.get("query_rope"),
              key_rope=inp.get("key_rope"), scale=case.scale_value, block_size=case.block, layout=case.layout,
              sparse_mode=case.mode, deterministic=det)
    args_pos = (inp["query"], inp["key"], inp["value"], inp["sparse_indices"], inp["dout"], inp["out"],
                inp["softmax_max"], inp["softmax_sum"])
    ws_bytes = sfag.workspace_size(*args_pos, *outs[:3], dq_rope=outs[3], dk_rope=outs[4], **kw)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        sfag.backward(*args_pos, outputs=outs, workspace=ws, stream=stream, **kw)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sfag.profile_reset()
    sfag.profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    sfag.profile_enable(False)
    ms = start.elapsed_time(stop) / args.steps
    prof = sfag.profile_read()
    print(f"[bench] {args.steps} steps, {ms:.3f} ms/step; kernels: "
          + ", ".join(f"{k}={v[0] / v[1]:.3f}ms x{v[1] // args.steps}" for k, v in prof.items()),
          file=sys.stderr, flush=True)

    tflops = flops / (ms * 1e-3) / 1e12
    alg_bytes = _alg_bytes(case, n_pairs)
    # Dominant kernel and its algorithmic work per launch.
    dom = max(prof, key=lambda k: prof[k][0])
    dom_ms = prof[dom][0] / prof[dom][1]
    launches_per_step = prof[dom][1] / args.steps
    if dom == "row":
        unit_flops = 2 * (2 * (case.D + case.Dr) + case.D)       # S, dQ over D+Dr; dP over D
        achieved = n_pairs * case.G * unit_flops / launches_per_step / (dom_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s")
    elif dom == "col":
        unit_flops = 2 * (2 * case.D + case.Dr)                  # dK over D+Dr, dV over D
        achieved = n_pairs * case.G * unit_flops / launches_per_step / (dom_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        achieved = alg_bytes / launches_per_step / (dom_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = dom
    roof["kernel_ms"] = dom_ms

    line = {
        "metric": "sparse-attn bwd TFLOP/s + % bf16 MFMA peak (G=128) / % HBM peak (G<=16), 1 GPU",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded generator; stand-in softmax statistics)",
        "config": {"workload": case.name, "layout": case.layout, "B": case.B, "T1": case.T1, "T2": case.T2,
                   "N1": case.G, "D": case.D, "Dr": case.Dr, "K": case.K, "sparse_block": case.block,
                   "sparse_mode": case.mode, "deterministic": det, "valid_pairs": n_pairs},
        "mfma_frac": tflops / MFMA_PEAK_TFLOPS,
        "alg_GBs": alg_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac_alg": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms": {k: v[0] / v[1] for k, v in prof.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = _cpu_baseline(case, inp, seed, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
