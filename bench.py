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


def _alg_bytes(case, n_pairs, value_is_key=False):
    """No-reuse algorithmic bytes of one backward call (with value passed as
    the key tensor, the V row of a pair is the K row already gathered)."""
    e = 2
    G, D, Dr, T1, T2 = case.G, case.D, case.Dr, case.T1, case.T2
    per_token = G * (D + Dr) * e * 2 + G * D * e * 2 + G * 4 * 2 + G * 4 * 2 + case.Kent * 4
    per_pair = ((D + Dr) if value_is_key else (2 * D + Dr)) * e + (2 * D + Dr) * 4
    per_key = (2 * D + Dr) * 4 * 2 + (2 * D + Dr) * e
    return T1 * per_token + n_pairs * per_pair + T2 * per_key


# Algorithmic flops per valid (head, selected position) pair of each MFMA
# kernel: S over D+Dr and dP over D (sdp); dQ over D+Dr (dq); both (row);
# dK over D+Dr and dV over D (keyblock, col).
def _unit_flops(case, kernel):
    D, Dr = case.D, case.Dr
    return {"sdp": 2 * (2 * D + Dr), "dq": 2 * (D + Dr), "row": 2 * (3 * D + 2 * Dr), "fwd": 2 * (2 * D + Dr),
            "keyblock": 2 * (2 * D + Dr), "col": 2 * (2 * D + Dr)}.get(kernel)


def _kernel_bytes(case, kernel, n_pairs):
    """Algorithmic HBM bytes of one step of a kernel group: every operand read
    once and every result written once (no re-reads)."""
    e = 2
    G, D, Dr, T1, T2 = case.G, case.D, case.Dr, case.T1, case.T2
    if kernel == "row":
        # Q, Qrope, dO, stats, indices in; dQ, dQrope out; per pair the
        # gathered K|Krope|V row in and the 16-bit dS and P out.
        return (T1 * (G * (2 * (D + Dr) + D) * e + G * 12 + case.Kent * 4)
                + n_pairs * ((2 * D + Dr) * e + 2 * G * e))
    if kernel == "fwd":
        # Q, Qrope, indices in; out and the two statistics out; per pair the
        # gathered K|Krope|V row in.
        return T1 * (G * (2 * D + Dr) * e + G * 8 + case.Kent * 4) + n_pairs * (2 * D + Dr) * e
    if kernel == "keyblock":
        # per pair dS and P in; per token Q|Qrope and dO in; per key the fp32
        # dK|dKrope|dV partial out.
        return n_pairs * 2 * G * e + T1 * G * (2 * D + Dr) * e + T2 * (2 * D + Dr) * 4
    return _alg_bytes(case, n_pairs)


def _roofline(case, kernel, kernel_ms, launches_per_step, n_pairs):
    uf = _unit_flops(case, kernel)
    if uf is not None and case.G >= 32:
        achieved = n_pairs * case.G * uf / launches_per_step / (kernel_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        achieved = _kernel_bytes(case, kernel, n_pairs) / launches_per_step / (kernel_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    return roof


def _traffic(case, kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter summary of
    this workload (FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy
    calibration), or None when there is none or the kernel's sources have
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{case.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    h = hashlib.sha256()
    for src in k["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != k["sources_sha256"]:
        return None
    return k["bytes_per_launch"]


# Kernel groups of the timing API and the kernels (by demangled name) and
# sources each one stands for.
_CSRC = "top_sparse_attention_sfag_amd/csrc/"
_COMMON = [_CSRC + "sfag_kernels.h", _CSRC + "sfag_device.h", _CSRC + "sfag_plan.h",
           "top_sparse_attention_sfag_amd/build.py"]
_GROUPS = {
    "sdp": (r"k_sdp<", [_CSRC + "sfag_sdp.hip"]),
    "dq": (r"k_dq<", [_CSRC + "sfag_sdp.hip"]),
    "row": (r"k_row<", [_CSRC + "sfag_row.hip"]),
    "keyblock": (r"k_keyblock<", [_CSRC + "sfag_keyblock.hip"]),
    "transpose": (r"k_transpose", [_CSRC + "sfag_keyblock.hip"]),
    "col": (r"k_col<", [_CSRC + "sfag_mfma.hip"]),
    "fwd": (r"k_fwd<", [_CSRC + "sfag_fwd.hip"]),
}


def _read_csvs(root, suffix):
    import csv
    rows = []
    for dp, _dn, fn in os.walk(root):
        for f in fn:
            if f.endswith(suffix):
                with open(os.path.join(dp, f), newline="") as fh:
                    rows += list(csv.DictReader(fh))
    return rows


def _summarize_profiles(d, config, calib_mb):
    """Turn rocprofv3 CSV output (``-f csv``) into the committed summaries:
    profiles/<workload>_kernel_stats.txt (kernel trace statistics) and
    profiles/traffic_<workload>.json (HBM bytes per launch from FETCH_SIZE
    and WRITE_SIZE, scaled by what the same counters read for one plain
    elementwise copy of ``calib_mb`` MiB)."""
    import hashlib
    import re

    import sfag_inputs as si
    case = si.CONFIGS[config]
    cmds = open(os.path.join(d, "commands.txt")).read().strip() if os.path.exists(
        os.path.join(d, "commands.txt")) else "(commands not recorded)"
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)

    stats = _read_csvs(os.path.join(d, "trace"), "kernel_stats.csv")
    lines = [f"# rocprofv3 kernel statistics: {case.name}", "",
             "Commands (from the repository root; OUT is an output directory):", "", cmds,
             f"python3 bench.py --summarize-profiles $OUT --config {config} --calib-copy-mb {calib_mb}", "",
             f"{'kernel':<72} {'calls':>6} {'avg us':>10} {'total ms':>10} {'%':>6}"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        if "sfag" not in name:
            continue
        lines.append(f"{name[:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:>10.3f} {float(r['Percentage']):>6.2f}")
    with open(os.path.join(out_dir, f"{case.name}_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(kind):
        acc = {}
        for r in _read_csvs(os.path.join(d, kind), "counter_collection.csv"):
            if r.get("Counter_Name") not in ("FETCH_SIZE", "WRITE_SIZE"):
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    fetch, write = per_kernel("fetch"), per_kernel("write")
    traffic = {"workload": case.name, "commands": cmds, "calibration": None, "kernels": {}}
    if calib_mb:
        # the calibration copy: the elementwise add that bench.py launches
        cand = [(max(v), k) for k, v in fetch.items() if "CUDAFunctorOnSelf_add<int>" in k]
        wc = [(max(v), k) for k, v in write.items() if "CUDAFunctorOnSelf_add<int>" in k]
        if cand and wc:
            kib = calib_mb * 1024.0
            ff, fk = max(cand)
            wf, wk = max(wc)
            traffic["calibration"] = dict(copy_MiB=calib_mb, kernel=fk[:120], fetch_KiB=ff, write_KiB=wf,
                                          fetch_factor=kib / ff, write_factor=kib / wf)
    cal = traffic["calibration"] or dict(fetch_factor=1.0, write_factor=1.0)
    for g, (pat, srcs) in _GROUPS.items():
        fv = [v for k, vs in fetch.items() if re.search(pat, k) for v in vs]
        wv = [v for k, vs in write.items() if re.search(pat, k) for v in vs]
        if not fv or not wv:
            continue
        h = hashlib.sha256()
        for src in srcs + _COMMON:
            with open(os.path.join(ROOT, src), "rb") as fh:
                h.update(fh.read())
        fb = sum(fv) / len(fv) * 1024 * cal["fetch_factor"]
        wb = sum(wv) / len(wv) * 1024 * cal["write_factor"]
        traffic["kernels"][g] = dict(dispatches=len(fv), fetch_bytes=fb, write_bytes=wb, bytes_per_launch=fb + wb,
                                     sources=srcs + _COMMON, sources_sha256=h.hexdigest())
    with open(os.path.join(out_dir, f"traffic_{case.name}.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    print("\n".join(lines))
    print(json.dumps({g: round(v["bytes_per_launch"] / 1e9, 3) for g, v in traffic["kernels"].items()}))
    return 0


def _cpu_baseline(case, inp, seed, target_s=15.0, forward=False):
    """The oracle as it stands, on one host thread, over a seeded sample of
    tokens: each sampled token's full backward (its dQ row and its dK/dV
    scatter), or its forward with ``forward``.  Batches double in size until
    about ``target_s`` seconds."""
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
            if forward:
                orc.forward(sub["q"], k, v, sub["qr"], kr, sub["idx"], g, case.block, case.mode, case.scale_value)
            else:
                orc.backward(sub["q"], k, v, sub["qr"], kr, sub["idx"], sub["dO"], sub["O"], sub["m"], sub["l"], g,
                             case.block, case.mode, case.scale_value)
            used += time.perf_counter() - t0
            rows = orc.decode(sub["idx"], case.block, case.mode, g)
            flops += (int((rows >= 0).sum()) * G * 2 * (2 * D + Dr) if forward else orc.flops(rows, G, D, Dr))
            done += len(sel)
            batch *= 2
    return dict(value=flops / used / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                sample=(f"{done} seeded tokens of the same workload, each token's full "
                        + ("forward" if forward else "backward (dQ row and dK/dV scatter)")
                        + f", float64 NumPy on one thread, {used:.1f} s"))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2, help="workload number (1-5); 2 is the headline")
    ap.add_argument("--deterministic", choices=("config", "true", "false"), default="config")
    ap.add_argument("--pass", dest="which", choices=("backward", "forward"), default="backward",
                    help="time the backward pass (the headline) or the forward pass that feeds it")
    ap.add_argument("--value-is-key", action="store_true",
                    help="pass the key tensor as value too (the operator page's supported case)")
    ap.add_argument("--dtype", choices=("config", "bf16", "fp16"), default="config",
                    help="input/output dtype (default: the workload's own)")
    ap.add_argument("--band", metavar="PRE,NEXT",
                    help="replace the workload's indices with a band (sliding-window / dense) selection made by "
                         "sfag_band_indices: key positions d-PRE..d+NEXT of the bottom-right diagonal d")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="summarize rocprofv3 CSV output under DIR/{trace,fetch,write} into profiles/ and exit")
    args = ap.parse_args(argv)
    if args.summarize_profiles:
        return _summarize_profiles(args.summarize_profiles, args.config, args.calib_copy_mb)
    if args.gpus != 1:
        print("bench.py measures a single GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch

    import sfag_inputs as si
    import top_sparse_attention_sfag_amd as sfag

    case = si.CONFIGS[args.config]
    if args.dtype != "config" and args.dtype != case.dtype:
        case = case.replace(name=f"{case.name}_as_{args.dtype}", dtype=args.dtype)
    band = None
    if args.band:
        band = tuple(int(x) for x in args.band.split(","))
        max_lk = case.S2 if case.layout == "BSND" else max(case.seqlens_kv)
        kb = sfag.band_entries(max_lk, band[0], band[1], case.block)
        case = case.replace(name=f"{case.name}_band_pre{band[0]}_next{band[1]}", K=kb, index_rule="uniform")
    det = case.deterministic if args.deterministic == "config" else args.deterministic == "true"
    seed = si.seed_for(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {case.name} on {dev}", file=sys.stderr, flush=True)
    inp = si.make_inputs(case, seed, device=dev)
    if band is not None:
        shape = tuple(inp["sparse_indices"].shape)
        kw_b = dict(pre_tokens=band[0], next_tokens=band[1], block_size=case.block, layout=case.layout, K=case.K)
        if case.layout == "BSND":
            kw_b.update(B=case.B, S1=case.S1, S2=case.S2, device=dev)
        else:
            kw_b.update(seqlens_q=inp["seqlens_q"], seqlens_kv=inp["seqlens_kv"])
        inp["sparse_indices"] = sfag.band_indices(**kw_b).reshape(shape)
    if args.value_is_key:
        inp["value"] = inp["key"]
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

    if args.which == "forward":
        # out / softmaxMax / softmaxSum written into the input tensors' copies
        fouts = (torch.empty_like(inp["out"]), torch.empty_like(inp["softmax_max"]),
                 torch.empty_like(inp["softmax_sum"]))
        fws = torch.empty(case.T1 * (case.Kent * case.block + 1) * 4 + 4096, dtype=torch.uint8, device=dev)
        fkw = dict(seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"),
                   query_rope=inp.get("query_rope"), key_rope=inp.get("key_rope"), scale=case.scale_value,
                   block_size=case.block, layout=case.layout, sparse_mode=case.mode)
        flops = n_pairs * case.G * 2 * (2 * case.D + case.Dr)

        def step():  # noqa: F811
            sfag.forward(inp["query"], inp["key"], inp["value"], inp["sparse_indices"], outputs=fouts,
                         workspace=fws, stream=stream, **fkw)

    if args.calib_copy_mb:
        # one elementwise kernel that reads and writes calib_copy_mb MiB each
        src = torch.ones((args.calib_copy_mb << 20) // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst
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
    alg_bytes = (_alg_bytes(case, n_pairs, args.value_is_key) if args.which == "backward"
                 else _kernel_bytes(case, "fwd", n_pairs))
    # Dominant kernel and its algorithmic work per launch.
    dom = max(prof, key=lambda k: prof[k][0])
    dom_ms = prof[dom][0] / prof[dom][1]
    launches_per_step = prof[dom][1] / args.steps
    roof = _roofline(case, dom, dom_ms, launches_per_step, n_pairs)
    roof["traffic"] = _traffic(case, dom)
    roof["kernel"] = dom
    roof["kernel_ms"] = dom_ms

    line = {
        "metric": ("sparse-attn bwd TFLOP/s + % bf16 MFMA peak (G=128) / % HBM peak (G<=16), 1 GPU"
                   if args.which == "backward" else "sparse-attn fwd TFLOP/s (forward pass), 1 GPU"),
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
                   "sparse_mode": case.mode, "deterministic": det, "valid_pairs": n_pairs,
                   "value_is_key": bool(args.value_is_key)},
        "mfma_frac": tflops / MFMA_PEAK_TFLOPS,
        "alg_GBs": alg_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac_alg": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms": {k: v[0] / v[1] for k, v in prof.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = _cpu_baseline(case, inp, seed, args.cpu_seconds, forward=args.which == "forward")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
