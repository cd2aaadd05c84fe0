"""Benchmark of one RBS prefill-attention layer on one MI355X.

A step is one pass of the hot path over the 128K workload: block statistics
(rbs_block_stats), dual-branch selection into CSR lists (rbs_select) and
block-sparse attention over the selected blocks (blocksparse_attn_fwd), all
on torch's current stream with inputs already resident in HBM.

Prints one JSON line. `value` is effective TFLOP/s of the whole step: the
attention flops on the selected blocks (4*D per admitted (query, key) pair,
counted from the emitted CSR) divided by the step time. `ms_per_step` is
ms/layer. `roofline` covers the dominant kernel (attention) against the
bf16 matrix-core peak; `phases` holds per-kernel HIP-event times and the
stats+select HBM fraction; `cpu_baseline` times the float64 CPU oracle on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu] [--no-extras]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 flop/clk)
FP8_PEAK_TFLOPS = 5033.2       # MI355X dense fp8 matrix-core peak (256 CU x 2.4 GHz x 8192 flop/clk)
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
METRIC = "block-sparse prefill attn ms/layer + effective TFLOP/s (% bf16 peak) at 128K"


def selected_pairs(row_ptr: np.ndarray, col_idx: np.ndarray, S: int, B: int, Hkv: int) -> int:
    """(query token, key token) pairs one query head admits, summed over KV
    groups: full blocks below the diagonal, the causal triangle on it."""
    nb = -(-S // B)
    rows = np.repeat(np.arange(Hkv * nb), np.diff(row_ptr))
    i = rows % nb
    j = col_idx.astype(np.int64)
    qlen = np.minimum(S, (i + 1) * B) - i * B
    klen = np.minimum(S, (j + 1) * B) - j * B
    full = np.where(j < i, qlen * klen, 0)
    diag = np.where(j == i, qlen * (qlen + 1) // 2, 0)
    return int(full.sum() + diag.sum())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense ratio and the Block-attention workload")
    ap.add_argument("--cpu-rows", type=int, default=448,
                    help="(KV head, query block) rows of the oracle's attention to time")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_rbs_amd as rbs
    from block_sparse_long_rbs_amd import device, inputs

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    w = inputs.mixture_bf16_128k()
    log(f"generated {w.name} in {time.perf_counter() - t_gen:.1f}s")
    t = device.upload(w)
    S, Hq, Hkv, D, B = w.seqlen, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block
    G = Hq // Hkv
    nb = w.n_blocks
    cap = rbs.rbs_select_capacity(Hkv, nb, w.keep_ratio_centroid, w.keep_ratio_rescue, w.sink)
    # the select workspace (about 9.5 MB at this size), allocated once outside the timed steps
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])

    def step():
        cen, rad, qr, qn = rbs.rbs_block_stats(t["q"], t["k"], B)
        rp, ci, _ = rbs.rbs_select(cen, rad, qr, qn, w.keep_ratio_centroid, w.keep_ratio_rescue,
                                   sink=w.sink, workspace=ws)
        rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, rp, ci, out=out)
        return rp, ci

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record(stream)
        cen, rad, qr, qn = rbs.rbs_block_stats(t["q"], t["k"], B)
        ev[s][1].record(stream)
        rp, ci, _ = rbs.rbs_select(cen, rad, qr, qn, w.keep_ratio_centroid, w.keep_ratio_rescue,
                                   sink=w.sink, workspace=ws)
        ev[s][2].record(stream)
        rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, rp, ci, out=out)
        ev[s][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    per = {name: np.array([ev[s][a].elapsed_time(ev[s][a + 1]) for s in range(K)])
           for a, name in enumerate(("stats", "select", "attn"))}
    t_attn = float(per["attn"].mean())
    # stats and select again, cold: a 512 MB buffer is read before each pair so
    # that neither L2 nor the 256 MB MALL holds Q, K or the statistics (a read
    # sweep, not a write: dirty lines left by a write would be written back to
    # HBM during the timed stats pass)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    flush_sum = torch.zeros((), dtype=torch.float32, device="cuda")
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for s_ in range(K):
        torch.sum(flush, dim=0, out=flush_sum)
        evc[s_][0].record(stream)
        cen, rad, qr, qn = rbs.rbs_block_stats(t["q"], t["k"], B)
        evc[s_][1].record(stream)
        rbs.rbs_select(cen, rad, qr, qn, w.keep_ratio_centroid, w.keep_ratio_rescue,
                       sink=w.sink, workspace=ws)
        evc[s_][2].record(stream)
    torch.cuda.synchronize()
    del flush, flush_sum
    cold = {name: np.array([evc[s_][a].elapsed_time(evc[s_][a + 1]) for s_ in range(K)])
            for a, name in enumerate(("stats", "select"))}
    t_stats, t_sel = float(cold["stats"].mean()), float(cold["select"].mean())
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    pairs = selected_pairs(rp_h, ci_h, S, B, Hkv) * G
    flops = 4.0 * D * pairs
    attn_tflops = flops / (t_attn * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    stats_bytes = S * (Hq + Hkv) * D * 2 + 2 * Hkv * nb * (D + 1) * 4
    select_bytes = 2 * Hkv * nb * (D + 1) * 4 + (Hkv * nb + 1) * 4 + int(rp_h[-1]) * 4
    log(f"step {ms_step:.3f} ms: stats {per['stats'].mean():.3f} select {per['select'].mean():.3f} "
        f"attn {t_attn:.3f} ms; attention {attn_tflops:.1f} TFLOP/s; cold stats {t_stats:.3f} "
        f"select {t_sel:.3f} ms")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seqlen": S, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "block": B, "keep_ratio_per_branch": w.keep_ratio_centroid,
                   "sink": w.sink, "beta": "derived", "seed": w.seed},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel<false> (CSR tiles)",
                     "achieved": round(attn_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": counted_traffic()},
        "phases": {
            "stats_ms": round(t_stats, 4), "select_ms": round(t_sel, 4),
            "attn_ms": round(t_attn, 4),
            "timing": "stats_ms and select_ms cold (512 MB read before each pair); "
                      "attn_ms and the *_in_step figures back to back inside the timed steps",
            "stats_ms_in_step": round(float(per["stats"].mean()), 4),
            "select_ms_in_step": round(float(per["select"].mean()), 4),
            "attn_flops": flops, "selected_pairs_per_head": pairs // G,
            "csr_nnz": int(rp_h[-1]),
            "stats_gbs": round(stats_bytes / (t_stats * 1e-3) / 1e9, 1),
            "stats_hbm_frac": round(stats_bytes / (t_stats * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stats_select_hbm_frac": round((stats_bytes + select_bytes) /
                                           ((t_stats + t_sel) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "select_gbs": round(select_bytes / (t_sel * 1e-3) / 1e9, 1),
            "select_hbm_frac": round(select_bytes / (t_sel * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "select_bound": "latency (three dependent kernels over ~5 MB; not HBM bound)",
            "stats_bytes": stats_bytes, "select_bytes": select_bytes,
            "percentiles_ms": {n: {"p10": round(float(np.percentile(v, 10)), 4),
                                   "median": round(float(np.median(v)), 4),
                                   "p90": round(float(np.percentile(v, 90)), 4)}
                               for n, v in (("stats", cold["stats"]), ("select", cold["select"]),
                                            ("attn", per["attn"]))},
        },
    }

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_extras:
        # dense causal attention through the same kernel (keep-ratio 1) for the sparse/dense ratio
        rows = [np.arange(i + 1, dtype=np.int32) for _ in range(Hkv) for i in range(nb)]
        rpd = np.zeros(Hkv * nb + 1, np.int64)
        np.cumsum([len(r) for r in rows], out=rpd[1:])
        rpd_t = torch.from_numpy(rpd.astype(np.int32)).cuda()
        cid_t = torch.from_numpy(np.concatenate(rows)).cuda()
        rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, rpd_t, cid_t, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(2):
            rbs.blocksparse_attn_fwd(t["q"], t["k"], t["v"], B, rpd_t, cid_t, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        t_dense = e0.elapsed_time(e1) / 2
        dense_flops = 4.0 * D * Hq * (S * (S + 1) // 2)
        result["dense_reference"] = {
            "attn_ms": round(t_dense, 3),
            "tflops": round(dense_flops / (t_dense * 1e-3) / 1e12, 1),
            "sparse_over_dense_speedup": round(t_dense / t_attn, 2),
        }
        log(f"dense causal attention {t_dense:.2f} ms -> speedup {t_dense / t_attn:.2f}x")
        del rpd_t, cid_t
        # shared-query execution (neighbouring query blocks over the union of
        # their lists) on the step's own lists, against the standard entry
        for _ in range(2):
            rbs.blocksparse_attn_fwd_shared_query(t["q"], t["k"], t["v"], B, rp, ci, out=out)
        e0.record(stream)
        for _ in range(5):
            rbs.blocksparse_attn_fwd_shared_query(t["q"], t["k"], t["v"], B, rp, ci, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        t_sq = e0.elapsed_time(e1) / 5
        result["shared_query_execution"] = {
            "attn_ms": round(t_sq, 4), "tflops": round(flops / (t_sq * 1e-3) / 1e12, 1),
            "time_over_standard_entry": round(t_sq / t_attn, 3),
            "note": "same lists and result; query blocks 2p, 2p+1 share key tiles in one workgroup"}
        log(f"shared-query execution {t_sq:.3f} ms ({t_sq / t_attn:.2f}x the standard entry)")
        # per-query-head selection (the other reading of the representative
        # query): one block list per query head, same keep ratios
        wsh = torch.empty(96 << 20, dtype=torch.uint8, device="cuda")
        outh = torch.empty_like(t["q"])

        def step_per_head():
            st_h = rbs.rbs_block_stats_per_head(t["q"], t["k"], B)
            rp_, ci_, _ = rbs.rbs_select_per_head(*st_h, w.keep_ratio_centroid,
                                                  w.keep_ratio_rescue, sink=w.sink, workspace=wsh)
            rbs.blocksparse_attn_fwd_per_head(t["q"], t["k"], t["v"], B, rp_, ci_, out=outh)
            return rp_, ci_

        for _ in range(2):
            step_per_head()
        torch.cuda.synchronize()
        evh = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(5)]
        for s_ in range(5):
            evh[s_][0].record(stream)
            st_h = rbs.rbs_block_stats_per_head(t["q"], t["k"], B)
            evh[s_][1].record(stream)
            rp_h2, ci_h2, _ = rbs.rbs_select_per_head(*st_h, w.keep_ratio_centroid,
                                                      w.keep_ratio_rescue, sink=w.sink,
                                                      workspace=wsh)
            evh[s_][2].record(stream)
            rbs.blocksparse_attn_fwd_per_head(t["q"], t["k"], t["v"], B, rp_h2, ci_h2, out=outh)
            evh[s_][3].record(stream)
        torch.cuda.synchronize()
        ph = [float(np.mean([evh[s_][a].elapsed_time(evh[s_][a + 1]) for s_ in range(5)]))
              for a in range(3)]
        rph = rp_h2.cpu().numpy().astype(np.int64)
        cih = ci_h2[:int(rph[-1])].cpu().numpy()
        flops_h = 4.0 * D * selected_pairs(rph, cih, S, B, Hq)
        result["per_query_head_selection"] = {
            "stats_ms": round(ph[0], 4), "select_ms": round(ph[1], 4), "attn_ms": round(ph[2], 4),
            "attn_flops": flops_h, "attn_tflops": round(flops_h / (ph[2] * 1e-3) / 1e12, 1),
            "csr_nnz": int(rph[-1]),
            "attn_ms_over_group_reading": round(ph[2] / t_attn, 3),
        }
        log(f"per-query-head selection: stats {ph[0]:.3f} select {ph[1]:.3f} attn {ph[2]:.3f} ms "
            f"({flops_h / (ph[2] * 1e-3) / 1e12:.1f} TFLOP/s, {int(rph[-1])} CSR entries)")
        del wsh, outh
        # fp8 (E4M3) Q, K, V with per-tensor descales, on the same block lists
        f8 = inputs.fp8_inputs(w)
        t8 = device.upload_fp8(f8)
        fp8_args = (t8["q"], t8["k"], t8["v"], B, rp, ci, f8.q_descale, f8.k_descale,
                    f8.v_descale)
        for _ in range(3):
            rbs.blocksparse_attn_fwd_fp8(*fp8_args, out=out)
        e0.record(stream)
        for _ in range(10):
            rbs.blocksparse_attn_fwd_fp8(*fp8_args, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        t_f8 = e0.elapsed_time(e1) / 10
        tf_f8 = flops / (t_f8 * 1e-3) / 1e12
        result["fp8_e4m3_attention"] = {
            "attn_ms": round(t_f8, 4), "tflops": round(tf_f8, 1),
            "frac_of_fp8_peak": round(tf_f8 / FP8_PEAK_TFLOPS, 4),
            "fp8_peak_tflops": FP8_PEAK_TFLOPS,
            "speedup_over_bf16": round(t_attn / t_f8, 3),
            "inputs": "the bf16 workload quantised per tensor to E4M3 (largest magnitude -> 448)"}
        log(f"fp8 attention {t_f8:.3f} ms, {tf_f8:.1f} TFLOP/s "
            f"({tf_f8 / FP8_PEAK_TFLOPS * 100:.1f}% of the fp8 peak)")
        del f8, t8, fp8_args
        # Block-attention RAG workload
        wr = inputs.rag_bf16_31k()
        tr = device.upload(wr)
        outr = torch.empty_like(tr["q"])
        args_r = (tr["q"], tr["k"], tr["v"], wr.seg_start.tolist(), wr.k_rerotate.tolist(),
                  wr.rope_theta)
        wsr = torch.empty(max(1, rbs.block_mask_workspace_bytes(*args_r)), dtype=torch.uint8,
                          device="cuda")
        for _ in range(3):
            rbs.block_mask_attn_fwd(*args_r, out=outr, workspace=wsr)
        e0.record(stream)
        for _ in range(10):
            rbs.block_mask_attn_fwd(*args_r, out=outr, workspace=wsr)
        e1.record(stream)
        torch.cuda.synchronize()
        t_bm = e0.elapsed_time(e1) / 10
        seg = wr.seg_start
        pairs_bm = 0
        for p in range(len(seg) - 1):
            L = int(seg[p + 1] - seg[p])
            lo = 0 if p == len(seg) - 2 else int(seg[p])
            pairs_bm += L * (int(seg[p]) - lo) + L * (L + 1) // 2
        fl_bm = 4.0 * wr.head_dim * wr.n_q_heads * pairs_bm
        # inference mode: the final block only (its rows see every cached passage)
        s_last = int(seg[-2])
        wsf = torch.empty(max(1, rbs.block_mask_workspace_bytes(*args_r, q_row_begin=s_last)),
                          dtype=torch.uint8, device="cuda")
        for _ in range(3):
            rbs.block_mask_attn_fwd(*args_r, q_row_begin=s_last, out=outr, workspace=wsf)
        e0.record(stream)
        for _ in range(10):
            rbs.block_mask_attn_fwd(*args_r, q_row_begin=s_last, out=outr, workspace=wsf)
        e1.record(stream)
        torch.cuda.synchronize()
        t_fin = e0.elapsed_time(e1) / 10
        Lf = int(seg[-1]) - s_last
        fl_fin = 4.0 * wr.head_dim * wr.n_q_heads * (Lf * s_last + Lf * (Lf + 1) // 2)
        result["block_mask_rag_31k"] = {
            "attn_ms": round(t_bm, 4), "tflops": round(fl_bm / (t_bm * 1e-3) / 1e12, 1),
            "flops": fl_bm,
            "final_block_only": {"attn_ms": round(t_fin, 4),
                                 "tflops": round(fl_fin / (t_fin * 1e-3) / 1e12, 1),
                                 "flops": fl_fin}}
        log(f"block-mask RAG 31K: {t_bm:.3f} ms, {fl_bm / (t_bm * 1e-3) / 1e12:.1f} TFLOP/s; "
            f"final block only {t_fin:.3f} ms, {fl_fin / (t_fin * 1e-3) / 1e12:.1f} TFLOP/s")
        del tr, outr, wsr, wsf

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, flops, args.cpu_rows, log)
    print(json.dumps(result), flush=True)


def counted_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB copy), or None when
    the kernel source has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "attn_bf16_csr_mixture_128k_pmc.md")
    csrc = os.path.join(ROOT, "block_sparse_long_rbs_amd", "csrc")
    try:
        text = open(path).read()
        h = hashlib.sha256()
        for name in ("attn_bf16.hip", "attn_tiles.h"):   # the kernel's sources, in this order
            h.update(open(os.path.join(csrc, name), "rb").read())
        sha = h.hexdigest()
    except OSError:
        return None
    m = re.search(r"source_sha256: ([0-9a-f]{64}).*?hbm_bytes_per_launch: (\d+)", text, re.S)
    if not m or m.group(1) != sha:
        return None
    return int(m.group(2))


def cpu_baseline(w, flops_total, n_rows, log):
    """The float64 oracle on the host cores: stats and selection over the full
    workload, attention on n_rows sampled (KV head, query block) rows,
    extrapolated to the whole layer by their share of the attention flops."""
    from oracle import rbs_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas = [(p.get("internal_api"), p.get("num_threads")) for p in threadpool_info()
                if p.get("user_api") == "blas"]
    except ImportError:
        blas = []
    host_cores = len(os.sched_getaffinity(0))
    cores = max([n for _, n in blas if n] or [host_cores])
    t0 = time.perf_counter()
    c, r, qr, qn = orc.block_stats(w.q, w.k, w.n_kv_heads, w.block)
    t_stats = time.perf_counter() - t0
    t0 = time.perf_counter()
    sel = orc.select(c, r, qr, qn, orc.derive_beta(r), w.keep_ratio_centroid,
                     w.keep_ratio_rescue, w.sink)
    t_sel = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    nb = w.n_blocks
    all_rows = [(g, i) for g in range(w.n_kv_heads) for i in range(nb)]
    rows = [all_rows[k] for k in rng.choice(len(all_rows), size=n_rows, replace=False)]
    t0 = time.perf_counter()
    orc.blocksparse_attention(w.q, w.k, w.v, w.block, sel.row_ptr, sel.col_idx, rows=rows)
    t_attn_sample = time.perf_counter() - t0
    sub_ptr = [0]
    sub_idx = []
    for g, i in rows:
        rr = g * nb + i
        blk = sel.col_idx[sel.row_ptr[rr]:sel.row_ptr[rr + 1]]
        sub_idx.extend(blk.tolist())
        sub_ptr.append(len(sub_idx))
    # flops of the sampled rows
    fl = 0
    for (g, i), a, b in zip(rows, sub_ptr[:-1], sub_ptr[1:]):
        for j in sub_idx[a:b]:
            L = min(w.seqlen, (i + 1) * w.block) - i * w.block
            fl += (L * L if j < i else L * (L + 1) // 2)
    fl *= 4.0 * w.head_dim * w.group
    t_attn_full = t_attn_sample * flops_total / max(fl, 1.0)
    t_total = t_stats + t_sel + t_attn_full
    val = flops_total / t_total / 1e12
    log(f"cpu oracle: stats {t_stats:.1f}s select {t_sel:.1f}s attention sample {t_attn_sample:.1f}s "
        f"-> {t_total:.0f}s per layer ({val:.4f} TFLOP/s)")
    return {"value": round(val, 6), "unit": "TFLOP/s", "cores": cores, "host_cores": host_cores,
            "cores_note": "cores = BLAS threads the oracle ran with; host_cores = CPUs in the "
                          "process's affinity set",
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle on the same 128K inputs: block stats and selection "
                       f"over all {w.n_kv_heads * nb} rows ({t_stats:.1f}s + {t_sel:.1f}s), "
                       f"attention on {n_rows} random (KV head, query block) rows "
                       f"({t_attn_sample:.1f}s for {fl:.3g} flops), extrapolated by flops to "
                       f"the whole layer: {t_total:.0f}s per layer"),
            "seconds_per_layer": round(t_total, 1), "blas": blas}


if __name__ == "__main__":
    main()
