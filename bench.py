#!/usr/bin/env python3
"""Throughput of the sparse flash attention backward on one MI355X.

One step = one full backward call (index decode, Delta, accumulator fill, the
MFMA kernels, the dK/dV key-centric reduction, and the cast) over one batch of
synthetic inputs already resident in HBM.  The headline workload is the
DSA-style training shape: BSND, B=1, S1=S2=4096, N1=128 heads sharing one
key/value head, D=512 plus a 64-wide rope part, K=2048 causal top-k indices
(25% local window, 75% uniform), bf16.  By default the other four workloads
(4 heads x 128 tokens x top-1024 of 2048; TND 64 heads x 8192 varlen tokens;
16 heads x 2 x 16384 tokens x 512 blocks of 16, fp16, no rope; 128 heads x
32768 tokens x top-8192 Zipf, deterministic) are timed in the same run and
reported under "configs".

out / softmaxMax / softmaxSum come from the library's own forward pass over
the same inputs, outside the timed region.

Prints one JSON line with the whole-job TFLOP/s (5504 flop per valid
(head, selected position) pair, 5120 without rope), the roofline of the
dominant kernel measured with HIP events inside the timed region, HBM bytes
from the committed rocprofv3 counter summary when it matches the sources,
and the CPU oracle timed on a bounded sample of the same workload.
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
    once and every result written once (no re-reads; a key row gathered by
    many tokens counts once)."""
    e = 2
    G, D, Dr, T1, T2 = case.G, case.D, case.Dr, case.T1, case.T2
    if kernel == "row":
        # Q, Qrope, dO, stats, Delta, indices in; dQ, dQrope out; the K|Krope|V
        # tables in; per pair the 16-bit dS and P out.
        return (T1 * (G * (2 * (D + Dr) + D) * e + G * 12 + case.Kent * 4) + T2 * (2 * D + Dr) * e
                + n_pairs * 2 * G * e)
    if kernel == "fwd":
        # Q, Qrope, indices in; out and the two statistics out; the K|Krope|V
        # tables in.
        return T1 * (G * (2 * D + Dr) * e + G * 8 + case.Kent * 4) + T2 * (2 * D + Dr) * e
    if kernel == "keyblock":
        # per pair dS and P in; per token Q|Qrope and dO in; per key the fp32
        # dK|dKrope|dV partial out.
        return n_pairs * 2 * G * e + T1 * G * (2 * D + Dr) * e + T2 * (2 * D + Dr) * 4
    return _alg_bytes(case, n_pairs)


def _roofline(case, kernel, kernel_ms, launches_per_step, n_pairs):
    """Algorithmic work of one launch of ``kernel`` over its average duration:
    flops against the bf16/fp16 MFMA peak for the MFMA kernels at N1 >= 32,
    otherwise the bytes each operand needs once against the HBM peak."""
    uf = _unit_flops(case, kernel)
    if uf is not None and case.G >= 32:
        achieved = n_pairs * case.G * uf / launches_per_step / (kernel_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        achieved = _kernel_bytes(case, kernel, n_pairs) / launches_per_step / (kernel_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    return roof


# Kernel groups of the timing API and the kernels (by demangled name) each
# one stands for.
_GROUPS = {
    "sdp": r"k_sdp8?<", "dq": r"k_dq<", "row": r"k_row(16)?<", "keyblock": r"k_keyblock<",
    "col": r"k_col<", "fwd": r"k_fwd8?<", "kb_reduce": r"k_kb_reduce", "cast": r"k_cast<", "decode": r"k_decode",
    "delta": r"k_delta<",
}
_SOURCES = ["include/sfag.h", "top_sparse_attention_sfag_amd/build.py"]


def _sources_sha256():
    """One hash over every source the library is built from."""
    import hashlib
    csrc = os.path.join(ROOT, "top_sparse_attention_sfag_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)) + _SOURCES:
        path = os.path.join(csrc, f) if "/" not in f else os.path.join(ROOT, f)
        with open(path, "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _traffic_record(case):
    """The committed counter summary of this workload when it was taken from
    the current sources, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{case.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != _sources_sha256():
        return None
    return rec


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
    """Turn rocprofv3 CSV output (``-f csv``) under d/{trace,rd,wr,mfma} into
    the committed summaries:

    * profiles/<workload>_kernel_stats.txt: kernel trace statistics of the
      backward kernels, and, when d/mfma holds SQ_VALU_MFMA_BUSY_CYCLES and
      GRBM_GUI_ACTIVE, each kernel's MFMA-busy fraction (busy cycles summed
      over the 1024 SIMDs over 1024 x its active cycles);
    * profiles/traffic_<workload>.json: HBM-side bytes per launch and per step
      from the TCC-to-memory request counters, read bytes = 32 x
      TCC_EA0_RDREQ_32B + 64 x TCC_EA0_RDREQ_64B + 128 x TCC_EA0_RDREQ_128B
      and write bytes = 64 x TCC_EA0_WRREQ_64B + 32 x (TCC_EA0_WRREQ -
      TCC_EA0_WRREQ_64B) (summed over every TCC instance); the elementwise
      copy of ``calib_mb`` MiB and the read-only sum over the same tensor that
      bench.py launches first are recorded beside them as a check.

    The backward steps of a counter run are the dispatches between the first
    and the last end-of-call kernel (k_cast, or on the key-block path the
    range reduction that writes the outputs: one per backward call; the
    forward pass and the index count that make the inputs run before the
    first call).  When d/trace also holds the per-dispatch kernel trace, the
    summary adds each kernel group's average over the last backward calls of
    the run, the serial pass that bench.py times kernels in when the library
    may overlap k_dq with the key-block kernels, next to the roofline kernel
    time bench.py printed in that run (d/trace.log)."""
    import re
    from collections import defaultdict

    import sfag_inputs as si
    case = si.CONFIGS[config]
    cmds = open(os.path.join(d, "commands.txt")).read().strip() if os.path.exists(
        os.path.join(d, "commands.txt")) else "(commands not recorded)"
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)

    def dispatches(kind):
        """{dispatch id: (kernel name, {counter: value})} of one counter run,
        each counter summed over the rows (instances) rocprofv3 reports."""
        out = {}
        for r in _read_csvs(os.path.join(d, kind), "counter_collection.csv"):
            i = int(r["Dispatch_Id"])
            name = r["Counter_Name"].replace("_sum", "")
            out.setdefault(i, (r["Kernel_Name"], defaultdict(float)))[1][name] += float(r["Counter_Value"])
        return out

    call_end = re.compile(r"k_cast<|k_kb_reduce<[^>]*true>")

    def window(disp):
        ids = sorted(i for i, (k, _c) in disp.items() if call_end.search(k))
        if len(ids) < 2:
            return {}, 0
        return {i: v for i, v in disp.items() if ids[0] < i <= ids[-1]}, len(ids) - 1

    rd_bytes = lambda c: 32 * c["TCC_EA0_RDREQ_32B"] + 64 * c["TCC_EA0_RDREQ_64B"] + 128 * c["TCC_EA0_RDREQ_128B"]
    wr_bytes = lambda c: 64 * c["TCC_EA0_WRREQ_64B"] + 32 * (c["TCC_EA0_WRREQ"] - c["TCC_EA0_WRREQ_64B"])

    # MFMA busy per kernel group: busy cycles summed over the 1024 SIMDs over
    # 1024 x the dispatch's active cycles (rocprofv3's MfmaUtil); the one
    # GRBM_GUI_ACTIVE value rocprofv3 reports adds up the active cycles of
    # the 8 XCDs' graphics blocks, so one XCD's share is an eighth of it
    mfma = {}
    md, nm = window(dispatches("mfma"))
    for g, pat in _GROUPS.items():
        rows = [c for k, c in md.values() if re.search(pat, k)]
        if rows and all("GRBM_GUI_ACTIVE" in c for c in rows):
            busy = sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for c in rows)
            act = sum(c["GRBM_GUI_ACTIVE"] for c in rows) / 8
            mfma[g] = busy / (act * 1024) if act else None

    stats = _read_csvs(os.path.join(d, "trace"), "kernel_stats.csv")
    lines = [f"# rocprofv3 kernel statistics: {case.name}", "",
             "Commands (from the repository root; OUT is an output directory):", "", cmds, "",
             f"{'kernel':<64} {'calls':>6} {'avg us':>10} {'total ms':>10} {'%':>6} {'MFMA busy':>9}"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        if "sfag" not in name:
            continue
        g = next((g for g, pat in _GROUPS.items() if re.search(pat, name)), None)
        mb = f"{mfma[g]:.3f}" if g in mfma and mfma[g] is not None else "-"
        lines.append(f"{name[:64]:<64} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:>10.3f} {float(r['Percentage']):>6.2f} {mb:>9}")
    # per-dispatch trace: each group's average over the serial pass (the last
    # n backward calls, n = bench.py's serial-pass length for the run's steps)
    trace = _read_csvs(os.path.join(d, "trace"), "kernel_trace.csv")
    if trace:
        rows = sorted((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                      for r in trace if "sfag" in r["Kernel_Name"])
        ends = [j for j, (_i, k, _t) in enumerate(rows) if call_end.search(k)]
        roof = None
        log = os.path.join(d, "trace.log")
        if os.path.exists(log):
            for line in open(log):
                if line.startswith("{"):
                    roof = json.loads(line).get("roofline")
        n = 5
        if len(ends) > n:
            sel = rows[ends[-n - 1] + 1: ends[-1] + 1]
            lines += ["", f"Serial pass (the last {n} backward calls of the trace run, each kernel alone on the GPU), "
                          "average per launch:"]
            for g, pat in _GROUPS.items():
                ts = [t for _i, k, t in sel if re.search(pat, k)]
                if ts:
                    lines.append(f"  {g:<10} {len(ts):>4} launches  {sum(ts) / len(ts) / 1e3:10.1f} us")
            if roof:
                lines.append(f"bench.py in the same run: roofline kernel {roof.get('kernel')}, "
                             f"{roof.get('kernel_ms', 0.0) * 1e3:.1f} us a launch ({roof.get('timing')})")
    with open(os.path.join(out_dir, f"{case.name}_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    rd_all, wr_all = dispatches("rd"), dispatches("wr")
    traffic = {"workload": case.name, "commands": cmds, "sources_sha256": _sources_sha256(), "calibration": None,
               "kernels": {}, "step": None, "mfma_busy": mfma or None}
    rf = wf = 1.0
    if calib_mb:
        # the counters see a fixed share of the TCC-to-memory requests: the
        # copy of known size gives the factor for reads and for writes, the
        # read-only sum a second reading of the read factor
        # (launched before any kernel of the library; a tensor above 2 GiB
        # runs as several dispatches of one kernel, so their counts add up)
        want = calib_mb * 1048576.0

        # the calibration runs first: its copy is every add dispatch before
        # the first reduction, its sum every reduction from there up to the
        # next add or library dispatch (the input generator's own adds and
        # reductions come later)
        def calib(disp):
            ids = sorted(disp)
            red = [i for i in ids if "reduce_kernel" in disp[i][0]]
            if not red:
                return [], []
            copy = [disp[i][1] for i in ids if i < red[0] and "CUDAFunctorOnSelf_add<" in disp[i][0]]
            run = []
            for i in ids[ids.index(red[0]):]:
                k = disp[i][0]
                if "CUDAFunctorOnSelf_add<" in k or "sfag" in k:
                    break
                if "reduce_kernel" in k:
                    run.append(disp[i][1])
            return copy, run
        cr, sr_ = calib(rd_all)
        cw, _ = calib(wr_all)
        cp_r = sum(rd_bytes(c) for c in cr)
        cp_w = sum(wr_bytes(c) for c in cw)
        sm_r = sum(rd_bytes(c) for c in sr_)
        cal = dict(bytes=want, copy_read=cp_r, copy_write=cp_w, sum_read=sm_r)
        if cp_r and cp_w:
            rf, wf = want / cp_r, want / cp_w
            cal.update(read_factor=rf, write_factor=wf, sum_read_factor=want / sm_r if sm_r else None)
        traffic["calibration"] = cal
    rd_bytes_raw, wr_bytes_raw = rd_bytes, wr_bytes
    rd_bytes = lambda c: rf * rd_bytes_raw(c)
    wr_bytes = lambda c: wf * wr_bytes_raw(c)
    rw, nr = window(rd_all)
    ww, nw = window(wr_all)
    for g, pat in _GROUPS.items():
        rv = [rd_bytes(c) for k, c in rw.values() if re.search(pat, k)]
        wv = [wr_bytes(c) for k, c in ww.values() if re.search(pat, k)]
        if not rv or not wv:
            continue
        traffic["kernels"][g] = dict(launches_per_step=len(rv) / nr, read_bytes=sum(rv) / len(rv),
                                     write_bytes=sum(wv) / len(wv),
                                     bytes_per_launch=sum(rv) / len(rv) + sum(wv) / len(wv))
    if nr and nw:
        sr = sum(rd_bytes(c) for k, c in rw.values() if "sfag" in k) / nr
        sw = sum(wr_bytes(c) for k, c in ww.values() if "sfag" in k) / nw
        traffic["step"] = dict(steps=nr, read_bytes=sr, write_bytes=sw, bytes=sr + sw)
    with open(os.path.join(out_dir, f"traffic_{case.name}.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    print("\n".join(lines))
    print(json.dumps({g: round(v["bytes_per_launch"] / 1e9, 3) for g, v in traffic["kernels"].items()}))
    if traffic["step"]:
        print(f"step bytes {traffic['step']['bytes'] / 1e9:.3f} GB")
    print("calibration", traffic["calibration"])
    return 0


def _host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return dict(model=model, logical_cpus=os.cpu_count(), usable_cpus=usable)


def _cpu_baseline(case, inp, seed, target_s=15.0, forward=False, threads=1):
    """The oracle as it stands, over a seeded sample of tokens: each sampled
    token's full backward (its dQ row and its dK/dV scatter), or its forward
    with ``forward``.  Batches double in size until about ``target_s``
    seconds.  With ``threads`` > 1 each batch is split over that many worker
    threads (one BLAS thread each; NumPy and torch release the interpreter
    lock inside their array operations), and the figure is the batch's flops
    over its wall time."""
    import concurrent.futures as cf

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
    def prepare(sel):
        ts = __import__("torch").as_tensor(sel)
        sub = {n: None if x is None else x[ts.to(x.device)].cpu() for n, x in full.items()}
        g = {n: (a[sel] if isinstance(a, np.ndarray) else a) for n, a in geom.items()}
        g["T1"] = len(sel)
        return sub, g

    def run(job):
        sub, g = job
        if forward:
            orc.forward(sub["q"], k, v, sub["qr"], kr, sub["idx"], g, case.block, case.mode, case.scale_value)
        else:
            orc.backward(sub["q"], k, v, sub["qr"], kr, sub["idx"], sub["dO"], sub["O"], sub["m"], sub["l"], g,
                         case.block, case.mode, case.scale_value)

    done, flops, used, batch = 0, 0, 0.0, 2 * threads
    with threadpool_limits(limits=1, user_api="blas"), cf.ThreadPoolExecutor(max_workers=threads) as pool:
        while used < target_s and done < T1:
            sel = np.sort(order[done:done + batch])
            jobs = [prepare(part) for part in np.array_split(sel, threads) if len(part)]
            t0 = time.perf_counter()
            list(pool.map(run, jobs))
            used += time.perf_counter() - t0
            for sub, g in jobs:
                rows = orc.decode(sub["idx"], case.block, case.mode, g)
                flops += (int((rows >= 0).sum()) * G * 2 * (2 * D + Dr) if forward else orc.flops(rows, G, D, Dr))
            done += len(sel)
            batch *= 2
    how = "one thread" if threads == 1 else f"{threads} worker threads of one BLAS thread each"
    return dict(value=flops / used / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=(f"{done} seeded tokens of the same workload, each token's full "
                        + ("forward" if forward else "backward (dQ row and dK/dV scatter)")
                        + f", float64 NumPy on {how}, {used:.1f} s"))


def _prepare(case, seed, dev, sfag, band=None, value_is_key=False):
    """Inputs of ``case`` on ``dev``, with out / softmaxMax / softmaxSum from
    the library's forward pass, and the number of valid pairs."""
    import torch

    import sfag_inputs as si
    inp = si.make_inputs(case, seed, device=dev)
    if band is not None:
        shape = tuple(inp["sparse_indices"].shape)
        kw_b = dict(pre_tokens=band[0], next_tokens=band[1], block_size=case.block, layout=case.layout, K=case.K)
        if case.layout == "BSND":
            kw_b.update(B=case.B, S1=case.S1, S2=case.S2, device=dev)
        else:
            kw_b.update(seqlens_q=inp["seqlens_q"], seqlens_kv=inp["seqlens_kv"])
        inp["sparse_indices"] = sfag.band_indices(**kw_b).reshape(shape)
    if value_is_key:
        inp["value"] = inp["key"]
    out, smax, ssum = sfag.forward(inp["query"], inp["key"], inp["value"], inp["sparse_indices"],
                                   seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"),
                                   query_rope=inp.get("query_rope"), key_rope=inp.get("key_rope"),
                                   scale=case.scale_value, block_size=case.block, layout=case.layout,
                                   sparse_mode=case.mode)
    inp.update(out=out, softmax_max=smax, softmax_sum=ssum)
    torch.cuda.synchronize()
    n_pairs, _ = _count_valid(case, inp, sfag)
    return inp, n_pairs


def _measure(case, inp, n_pairs, det, steps, warmup, sfag, which="backward", value_is_key=False, options=None):
    """Time ``steps`` calls after ``warmup`` (HIP events on the call's stream
    around the whole region and around each kernel group), and the roofline
    of the kernel group with the largest time per step.  When the call runs
    the dQ kernel on a second stream beside the key-block kernels, the
    per-kernel times for the roofline come from a separate serial pass."""
    import torch
    dev = inp["query"].device
    outs = (torch.empty_like(inp["query"]), torch.empty_like(inp["key"]), torch.empty_like(inp["value"]),
            torch.empty_like(inp["query_rope"]) if case.Dr else None,
            torch.empty_like(inp["key_rope"]) if case.Dr else None)
    kw = dict(seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"), query_rope=inp.get("query_rope"),
              key_rope=inp.get("key_rope"), scale=case.scale_value, block_size=case.block, layout=case.layout,
              sparse_mode=case.mode, deterministic=det)
    args_pos = (inp["query"], inp["key"], inp["value"], inp["sparse_indices"], inp["dout"], inp["out"],
                inp["softmax_max"], inp["softmax_sum"])
    stream = torch.cuda.current_stream(dev)
    if which == "forward":
        fouts = (torch.empty_like(inp["out"]), torch.empty_like(inp["softmax_max"]),
                 torch.empty_like(inp["softmax_sum"]))
        fkw = dict(seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"),
                   query_rope=inp.get("query_rope"), key_rope=inp.get("key_rope"), scale=case.scale_value,
                   block_size=case.block, layout=case.layout, sparse_mode=case.mode)
        fws = torch.empty(case.T1 * (case.Kent * case.block + 1) * 4 + (1 << 20), dtype=torch.uint8, device=dev)
        flops = n_pairs * case.G * 2 * (2 * case.D + case.Dr)

        def step(opts=None):
            sfag.forward(inp["query"], inp["key"], inp["value"], inp["sparse_indices"], outputs=fouts,
                         workspace=fws, stream=stream, **fkw)
        concurrent = False
    else:
        ws_bytes = sfag.workspace_size(*args_pos, *outs[:3], dq_rope=outs[3], dk_rope=outs[4], options=options, **kw)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        flops = n_pairs * case.G * 2 * (3 * (case.D + case.Dr) + 2 * case.D)

        def step(opts=options):
            sfag.backward(*args_pos, outputs=outs, workspace=ws, stream=stream, options=opts, **kw)
        # unless told to stay serial the library may run the dQ kernel on a
        # second stream beside the key-block kernels (see
        # sfag_options.concurrent; by default for 32 <= N1 < 128, and for 128
        # heads with short chunks): the per-kernel times that pick the
        # roofline kernel then come from a serial pass
        cc = (options or {}).get("concurrent", "auto")
        concurrent = cc != "off"

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    sfag.profile_reset()
    sfag.profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    sfag.profile_enable(False)
    ms = start.elapsed_time(stop) / steps
    prof = sfag.profile_read()
    nsteps_r = steps
    rprof = prof
    if concurrent:
        serial = dict(options or {}, concurrent="off")
        nsteps_r = max(2, min(steps, 5))
        sfag.profile_reset()
        sfag.profile_enable(True)
        for _ in range(nsteps_r):
            step(serial)
        torch.cuda.synchronize()
        sfag.profile_enable(False)
        rprof = sfag.profile_read()
    print(f"[bench] {case.name}: {steps} steps, {ms:.3f} ms/step; kernels: "
          + ", ".join(f"{k}={v[0] / v[1]:.3f}ms x{v[1] // steps}" for k, v in prof.items()),
          file=sys.stderr, flush=True)
    tflops = flops / (ms * 1e-3) / 1e12
    alg_bytes = (_alg_bytes(case, n_pairs, value_is_key) if which == "backward"
                 else _kernel_bytes(case, "fwd", n_pairs))
    # the roofline kernel: the largest time per step when every kernel runs
    # alone; its duration from the timed region unless it shares the GPU with
    # the second stream's kernels there
    dom = max(rprof, key=lambda k: rprof[k][0])
    overlapped = concurrent and dom in ("dq", "keyblock", "kb_sort")
    src = rprof if overlapped or dom not in prof else prof
    dom_ms = src[dom][0] / src[dom][1]
    launches_per_step = src[dom][1] / (nsteps_r if src is rprof else steps)
    timing = ("HIP events on the kernel's stream in a serial pass after the timed region (the default schedule "
              "may overlap it with the second stream)" if src is rprof and concurrent
              else "HIP events on the kernel's stream in the timed region")
    roof = _roofline(case, dom, dom_ms, launches_per_step, n_pairs)
    rec = _traffic_record(case) if which == "backward" and not value_is_key and options is None else None
    roof["traffic"] = rec["kernels"].get(dom, {}).get("bytes_per_launch") if rec else None
    roof["kernel"] = dom
    roof["kernel_ms"] = dom_ms
    roof["timing"] = timing
    if dom in ("row", "fwd"):
        # rate at which the kernel gathers selected K|Krope|V rows (from L2 and
        # the last-level cache, mostly): context for its HBM roofline
        rb = (case.D + case.Dr if value_is_key else 2 * case.D + case.Dr) * 2
        roof["gathered_rows_GBs"] = n_pairs * rb / launches_per_step / (dom_ms * 1e-3) / 1e9
    out = dict(workload=case.name, steps=steps, warmup=warmup, ms_per_step=ms, tflops=tflops,
               mfma_frac=tflops / MFMA_PEAK_TFLOPS, valid_pairs=n_pairs,
               alg_model_GBs=alg_bytes / (ms * 1e-3) / 1e9,
               kernels_ms={k: v[0] / v[1] for k, v in prof.items()}, roofline=roof)
    # counter-measured bytes of the step's L2 misses (TCC requests to the
    # memory fabric, served by the last-level cache or HBM: an upper bound on
    # the HBM bytes), from the committed summary of this workload when it was
    # taken from the current sources
    if rec and rec.get("step"):
        gbs = rec["step"]["bytes"] / (ms * 1e-3) / 1e9
        out.update(l2_miss_GB_per_step=rec["step"]["bytes"] / 1e9, l2_miss_GBs=gbs,
                   l2_miss_frac_of_hbm_peak=gbs / HBM_PEAK_GBS)
    else:
        out.update(l2_miss_GB_per_step=None, l2_miss_GBs=None, l2_miss_frac_of_hbm_peak=None)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=None,
                    help="time only this workload (1-5); by default 2 is the headline and 1, 3, 4, 5 follow")
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
    ap.add_argument("--concurrent", choices=("auto", "off", "on"), default="auto",
                    help="sfag_options.concurrent for the timed calls (default: the library's choice)")
    ap.add_argument("--token-path", choices=("auto", "fused", "split"), default="auto",
                    help="sfag_options.tokenPath for the timed calls (default: the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run one plain device copy and one read-only sum of this many MiB (counter "
                         "calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="summarize rocprofv3 CSV output under DIR/{trace,rd,wr,mfma} into profiles/ and exit")
    args = ap.parse_args(argv)
    if args.summarize_profiles:
        return _summarize_profiles(args.summarize_profiles, args.config or 2, args.calib_copy_mb)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import sfag_inputs as si
    import top_sparse_attention_sfag_amd as sfag

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mb:
        # one elementwise kernel that reads and writes calib_copy_mb MiB each,
        # and one reduction that only reads them
        src = torch.ones((args.calib_copy_mb << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        total = src.sum()   # float32: reduced as it is, no widened copy first
        torch.cuda.synchronize()
        del src, dst, total

    def case_of(cfg):
        case = si.CONFIGS[cfg]
        if args.dtype != "config" and args.dtype != case.dtype:
            case = case.replace(name=f"{case.name}_as_{args.dtype}", dtype=args.dtype)
        band = None
        if args.band:
            band = tuple(int(x) for x in args.band.split(","))
            max_lk = case.S2 if case.layout == "BSND" else max(case.seqlens_kv)
            kb = sfag.band_entries(max_lk, band[0], band[1], case.block)
            case = case.replace(name=f"{case.name}_band_pre{band[0]}_next{band[1]}", K=kb, index_rule="uniform")
        det = case.deterministic if args.deterministic == "config" else args.deterministic == "true"
        return case, band, det

    headline = args.config or 2
    sweep = [] if args.config else [1, 3, 4, 5]
    case, band, det = case_of(headline)
    seed = si.seed_for(headline)
    print(f"[bench] generating {case.name} on {dev}", file=sys.stderr, flush=True)
    inp, n_pairs = _prepare(case, seed, dev, sfag, band, args.value_is_key)
    opts = {}
    if args.concurrent != "auto":
        opts["concurrent"] = args.concurrent
    if args.token_path != "auto":
        opts["token_path"] = args.token_path
    opts = opts or None
    head = _measure(case, inp, n_pairs, det, args.steps, args.warmup, sfag, args.which, args.value_is_key, opts)

    line = {
        "metric": ("sparse-attn bwd TFLOP/s + % bf16 MFMA peak (G=128) / % HBM peak (G<=16), 1 GPU"
                   if args.which == "backward" else "sparse-attn fwd TFLOP/s (forward pass), 1 GPU"),
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded generator); out/softmaxMax/softmaxSum from the library's forward pass",
        "config": {"workload": case.name, "layout": case.layout, "B": case.B, "T1": case.T1, "T2": case.T2,
                   "N1": case.G, "D": case.D, "Dr": case.Dr, "K": case.K, "sparse_block": case.block,
                   "sparse_mode": case.mode, "deterministic": det, "valid_pairs": n_pairs,
                   "value_is_key": bool(args.value_is_key)},
        "mfma_frac": head["mfma_frac"],
        "alg_model_GBs": head["alg_model_GBs"],
        "l2_miss_GBs": head["l2_miss_GBs"],
        "l2_miss_frac_of_hbm_peak": head["l2_miss_frac_of_hbm_peak"],
        "kernels_ms": head["kernels_ms"],
        "roofline": head["roofline"],
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        host = _host_cpu()
        cb = _cpu_baseline(case, inp, seed, args.cpu_seconds, forward=args.which == "forward")
        cores = max(1, min(16, host["usable_cpus"] or 1))
        allc = _cpu_baseline(case, inp, seed, args.cpu_seconds / 2, forward=args.which == "forward", threads=cores)
        cb["host"] = host
        cb["all_cores"] = dict(value=allc["value"], unit=allc["unit"], cores=cores, sample=allc["sample"])
        line["cpu_baseline"] = cb
    del inp
    torch.cuda.empty_cache()
    if sweep:
        line["configs"] = {}
        for cfg in sweep:
            c, b, d = case_of(cfg)
            print(f"[bench] generating {c.name}", file=sys.stderr, flush=True)
            inp_c, n_c = _prepare(c, si.seed_for(cfg), dev, sfag, b, args.value_is_key)
            st = args.steps if cfg <= 3 else max(3, args.steps // 4)
            rec = _measure(c, inp_c, n_c, d, st, min(args.warmup, 2) if cfg > 3 else args.warmup, sfag, args.which,
                           args.value_is_key, opts)
            rec["config"] = {"layout": c.layout, "B": c.B, "T1": c.T1, "T2": c.T2, "N1": c.G, "D": c.D, "Dr": c.Dr,
                             "K": c.K, "sparse_block": c.block, "sparse_mode": c.mode, "deterministic": d,
                             "dtype": c.dtype}
            line["configs"][f"cfg{cfg}"] = rec
            del inp_c
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
