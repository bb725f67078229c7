"""Benchmark of one Spark-Attn layer on one MI355X.

A step is one pass of the whole layer -- spark_reblock (moments, square
roots, whitening, hierarchical split, gather + pooling), spark_select,
spark_summarize, spark_attn (fused exact + compressed attention with the
scatter) -- over the 768p workload: a 61x48x84 latent (245,952 tokens),
H=40, d=128, block 128, density 0.1 (top 193 of 1922 key blocks), bf16,
seeded synthetic clustered q/k (see block_sparse_attention_mahalanobis_amd/
workload.py).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the median layer latency in ms over the
timed steps (HIP events; lower is better);
the exact-branch MFMA fraction of the bf16 dense peak, per-stage times, the
attention kernel's roofline and the fp64 CPU oracle baseline ride along.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="full768", choices=["full768", "draft", "ref2va", "tiny"])
    p.add_argument("--ratio", type=float, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this size before timing (counter calibration)")
    p.add_argument("--cpu-sample-blocks", type=int, default=768,
                   help="query blocks of head 0 the oracle attends in the CPU baseline sample")
    p.add_argument("--layout", default="reblock", choices=["reblock", "q_reuse_k"],
                   help="token partition: separate query/key Spark-Reblock, or the key partition reused")
    p.add_argument("--sweep", action="store_true",
                   help="the density / noise sweep at the draft shape instead of the layer line")
    p.add_argument("--fp8", action="store_true",
                   help="attention logits from E4M3 operands (queries per row, keys per block)")
    p.add_argument("--context", action="store_true",
                   help="tokens from n_anchor on (the ref2va reference frames) are context tokens: "
                        "exact for every query, outside the video-block top-k")
    p.add_argument("--one-block", action="store_true",
                   help="one query block per attention workgroup (SPARK_ATTN_ONE_BLOCK) instead of the "
                        "paired schedule")
    return p.parse_args()


def load_inputs(w, torch, dtype, threads):
    """q, k, v [H, N, d] on cuda:0, generated head by head on the host."""
    from block_sparse_attention_mahalanobis_amd.workload import make_head
    H, N, d = w.H, w.N, w.d
    out = [torch.empty((H, N, d), dtype=dtype, device="cuda:0") for _ in range(3)]
    with ThreadPoolExecutor(threads) as ex:
        for h, arrs in enumerate(ex.map(lambda hh: make_head(w, hh), range(H))):
            for t, a in zip(out, arrs):
                t[h].copy_(torch.from_numpy(a).to(dtype))
    torch.cuda.synchronize()
    return out


def attn_flops(idx, N, b, d, Nv=None):
    """Algorithmic flops of the fused attention: 4 d per (query row, exact
    key) plus 4 d per (query row, unselected block summary).  With context
    tokens (Nv < N) every video row also takes the N - Nv context keys
    exactly and every context row all N keys."""
    Nv = N if Nv is None else Nv
    H, nb, k = idx.shape
    sizes = np.full(nb, b, dtype=np.int64)
    sizes[-1] = Nv - (nb - 1) * b
    keys_per_qblock = sizes[idx].sum(axis=2) + (N - Nv)      # [H, nb]
    exact = 4 * d * int((keys_per_qblock * sizes[None, :]).sum()) + 4 * d * H * (N - Nv) * N
    comp = 4 * d * int(H * Nv * (nb - k))
    return exact, comp


def split_rows_read(Nv, b, levels_global, root_fused=False):
    """Rows one side's global split levels read: the centroid, pole-A, pole-B
    and score passes over every group that splits (>= 2 blocks), except that
    below the root the centroid pass skips right children (a right child's
    sum is its parent's minus its sibling's), and with root_fused the root's
    centroid comes from the whitening pass (no read)."""
    def nrows(start, n):
        return min(Nv, (start + n) * b) - start * b
    groups, rows = [(0, -(-Nv // b), False)], 0
    for _ in range(levels_global):
        nxt = []
        for start, n, right in groups:
            if n < 2:
                continue
            rows += (3 if right or (root_fused and start == 0 and n == -(-Nv // b)) else 4) * nrows(start, n)
            nl = (n + 1) // 2
            nxt += [(start, nl, False), (start + nl, n - nl, True)]
        groups = nxt
    return rows


def reblock_bytes(H, N, d, b, es, levels_global, nb, sides=2, Nv=None):
    """Algorithmic HBM bytes of reblock + summaries (per layer); sides = 1
    for q_reuse_k (moments of q only, keys whitened and split).  With
    context tokens only the Nv video rows are whitened, split and summarised."""
    Nv = N if Nv is None else Nv
    vol = H * N * d * es                      # one [H, N, d] tensor
    volv = H * Nv * d * es                    # its video rows
    moments = sides * vol
    whiten = 2 * sides * volv
    fused = es == 2 and d == 128 and b == 128   # the whitening pass sums the root's blocks
    split = sides * (H * split_rows_read(Nv, b, levels_global, fused) * d * es + volv)   # + finisher
    gather = 6 * vol
    summ = 2 * volv
    return moments + whiten + split + gather + summ


def cpu_baseline(w, topk, sample_blocks, context=False):
    """The fp64 oracle as it stands, timed on this host: head 0 end to end
    (reblock of both sides, pooling, scores, top-k, summaries) plus the
    two-branch attention of `sample_blocks` query blocks (and, with context
    tokens, the dense rows of up to 1024 context queries), scaled to the
    whole layer (H heads, all query blocks and context rows)."""
    import oracle as O
    from block_sparse_attention_mahalanobis_amd.workload import make_head
    cores = len(os.sched_getaffinity(0))
    q, k, v = make_head(w, 0)
    b = w.block
    nv = w.n_anchor if context else w.N
    nb = O.n_blocks(nv, b)
    t0 = time.perf_counter()
    pq, pk = O.reblock_head(q, k, b, n_split=nv)
    qp, qbar = O.gather_pool(q[:nv], pq, b)
    kp, kbar = O.gather_pool(k[:nv], pk, b)
    vp = np.asarray(v[:nv], np.float64)[pk]
    S = O.block_scores(qbar, kbar)
    idx = O.select_topk(S, topk)
    ks, vs, beta = O.reweight_summaries(kp, vp, O.anchor_query(q, w.n_anchor), b)
    t1 = time.perf_counter()
    nsamp = min(sample_blocks, nb)
    O.sparse_attention(qp, kp, vp, idx, ks, vs, beta, b, qblocks=range(nsamp),
                       extra_k=k[nv:] if nv < w.N else None, extra_v=v[nv:] if nv < w.N else None)
    t2 = time.perf_counter()
    per_head = (t1 - t0) + (t2 - t1) * (nb / nsamp)
    extra = ""
    if nv < w.N:
        nc = w.N - nv
        ncs = min(1024, nc)
        O.dense_attention(q[nv:nv + ncs], k, v)
        t3 = time.perf_counter()
        per_head += (t3 - t2) * (nc / ncs)
        extra = f" + dense rows of {ncs}/{nc} context queries ({t3 - t2:.1f} s)"
    layer_ms = per_head * w.H * 1e3
    return {"value": round(layer_ms, 1), "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": (f"head 0 of {w.H}: full reblock/select/summaries ({t1 - t0:.1f} s) + attention "
                       f"of {nsamp}/{nb} query blocks ({t2 - t1:.1f} s){extra}, scaled to all blocks "
                       f"and x{w.H} heads; numpy fp64, BLAS threads = {cores}")}


def load_traffic(name, sources, key, kernel=None):
    """Measured HBM bytes from a committed rocprofv3 --pmc summary under
    profiles/, if it was taken on the current kernel sources and, where
    given, for the same kernel (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    h = hashlib.sha256()
    for src in sources:
        h.update(open(src, "rb").read())
    if rec.get("kernel_sha") != h.hexdigest()[:16]:
        return None
    if kernel is not None and rec.get("kernel") != kernel:
        return None
    return rec.get(key)


def sweep(args):
    """Density and noise sweep at the 16x24x42 draft shape (H=24, N=16,128):
    clustered and i.i.d. N(0,1) q/k, top-k ratio 0.1/0.2/0.3/1.0, Reblock,
    q_reuse_k (the key partition reused for the queries) and fixed
    consecutive blocks.  Per row: layer latency (HIP events around
    spark_layer, inputs resident) and, outside the timing, the mean
    attention-mass recall and log-mass error from spark_diagnostics.  One JSON
    line; not the headline measurement."""
    import torch

    from block_sparse_attention_mahalanobis_amd import _lib as L
    from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    w0 = WORKLOADS["sweep"]
    H, N, d, b = w0.H, w0.N, w0.d, w0.block
    nb = L.n_blocks(N, b)
    rows = []
    for iid in (False, True):
        w = w0.with_(iid=iid)
        q, k, v = load_inputs(w, torch, torch.bfloat16, threads)
        out = torch.empty_like(q)
        for ratio in (0.1, 0.2, 0.3, 1.0):
            topk = L.topk_from_ratio(ratio, nb)
            for layout in ("reblock", "q_reuse_k", "identity"):
                a = L.make_args(H, N, d, b, torch.bfloat16, None, layout)
                ws = torch.empty(max(L.workspace_bytes(a, L.OP_LAYER, topk), 256), dtype=torch.uint8,
                                 device="cuda:0")
                for _ in range(args.warmup):
                    L.spark_layer(q, k, v, b, topk, layout=layout, out=out, ws=ws)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    L.spark_layer(q, k, v, b, topk, layout=layout, out=out, ws=ws)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / args.steps
                del ws
                g = L.spark_reblock(q, k, v, b, layout=layout)
                idx = L.spark_select(g["qbar"], g["kbar"], topk, N, b)
                ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
                rec, lme = L.spark_diagnostics(g["q_p"], g["k_p"], idx, ks, bias, N, b)
                torch.cuda.synchronize()
                row = {"data": "iid" if iid else "clustered", "ratio": ratio, "topk": topk, "layout": layout,
                       "ms": round(ms, 3), "recall": round(float(rec.mean()), 4),
                       "log_mass_error": round(float(lme.mean()), 4)}
                log(json.dumps(row))
                rows.append(row)
                del g, idx, ks, vs, bias, rec, lme
        del q, k, v, out
    print(json.dumps({"metric": "density/noise sweep: layer latency (ms) and attention-mass recall, "
                                "Reblock vs q_reuse_k vs fixed blocks",
                      "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "data": "synthetic (seeded; clustered Gaussian mixture on the latent grid, or "
                              "i.i.d. N(0,1) q/k; v ~ N(0,1))",
                      "config": {"workload": "sweep", "H": H, "N": N, "d": d, "block": b, "n_blocks": nb,
                                 "summary": "reweight"},
                      "rows": rows}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU; multi-GPU runs are not part of "
                                   "this implementation (heads would shard with zero communication)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    import torch

    import block_sparse_attention_mahalanobis_amd as S
    from block_sparse_attention_mahalanobis_amd import _lib as L
    from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.lib()
    w = WORKLOADS[args.config]
    if args.ratio is not None:
        w = w.with_(ratio=args.ratio)
    dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    es = 2 if w.dtype == "bf16" else 4
    H, N, d, b = w.H, w.N, w.d, w.block
    ctx = args.context and w.n_anchor < N
    Nv, nb, nbt = L.geometry(N, b, w.n_anchor, ctx)
    topk = L.topk_from_ratio(w.ratio, nb)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    log(f"workload {w.name}: H={H} N={N} d={d} block={b} n_b={nb} topk={topk} dtype={w.dtype}"
        + (f"; context tokens {N - Nv} ({nbt - nb} blocks)" if ctx else ""))
    t = time.perf_counter()
    q, k, v = load_inputs(w, torch, dtype, threads)
    log(f"inputs resident ({time.perf_counter() - t:.1f} s)")

    # buffers and workspaces, allocated once
    Np = nbt * b
    dev = "cuda:0"
    perm_q = torch.empty((H, N), dtype=torch.int32, device=dev)
    perm_k = torch.empty((H, N), dtype=torch.int32, device=dev)
    q_p = torch.empty((H, Np, d), dtype=dtype, device=dev)
    k_p = torch.empty((H, Np, d), dtype=dtype, device=dev)
    v_pt = torch.empty((H, nbt, d, b), dtype=dtype, device=dev)
    qbar = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
    kbar = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
    anchor = torch.empty((H, d), dtype=torch.float32, device=dev)
    idx = torch.empty((H, nb, topk), dtype=torch.int32, device=dev)
    ksum = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
    vsum = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
    bias = torch.empty((H, nb), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    a = L.make_args(H, N, d, b, dtype, w.n_anchor, args.layout, context=ctx, fp8=args.fp8,
                    one_block=args.one_block)
    ws_r = L.workspace_bytes(a, L.OP_REBLOCK)
    ws_a = L.workspace_bytes(a, L.OP_ATTN)
    ws = torch.empty(max(ws_r, ws_a, 256), dtype=torch.uint8, device=dev)
    lib = L.lib()
    import ctypes
    P = L._ptr
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ab = ctypes.byref(a)

    def step(ev=None):
        if ev: ev[0].record(stream)
        L._check(lib.spark_reblock(ab, P(q), P(k), P(v), P(perm_q), P(perm_k), P(q_p), P(k_p), P(v_pt),
                                   P(qbar), P(kbar), P(anchor), P(ws), ws.numel(), sp), "spark_reblock")
        if ev: ev[1].record(stream)
        L._check(lib.spark_select(ab, P(qbar), P(kbar), None, topk, P(idx), None, sp), "spark_select")
        if ev: ev[2].record(stream)
        L._check(lib.spark_summarize(ab, P(k_p), P(v_pt), P(anchor), P(ksum), P(vsum), P(bias), sp),
                 "spark_summarize")
        if ev: ev[3].record(stream)
        L._check(lib.spark_attn(ab, P(q_p), P(k_p), P(v_pt), P(idx), topk, P(ksum), P(vsum), P(bias),
                                P(perm_q), P(out), P(ws), ws.numel(), sp), "spark_attn")
        if ev: ev[4].record(stream)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read + {n} bytes written")
        del src, dst
    for i in range(args.warmup):
        step()
        log(f"warmup {i + 1}/{args.warmup}")
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms
    per_step = np.array([e[0].elapsed_time(e[4]) for e in evs])                        # ms
    # the median over the timed steps (HIP events on the launch stream); the
    # wall-clock mean over the same steps rides along
    layer_ms = float(np.median(per_step))
    wall_ms = wall * 1e3 / args.steps
    st_mean = np.median(stages, axis=0)
    log(f"layer {layer_ms:.2f} ms (median of {args.steps}; wall mean {wall_ms:.2f}); reblock {st_mean[0]:.2f} "
        f"select {st_mean[1]:.2f} summarize {st_mean[2]:.2f} attn {st_mean[3]:.2f} ms")
    peak_meas = L.mfma_peak_tflops()
    log(f"measured bf16 MFMA rate (register-only loop): {peak_meas:.0f} TFLOP/s")

    exact, comp = attn_flops(idx.cpu().numpy(), N, b, d, Nv)
    attn_s = st_mean[3] * 1e-3
    exact_tf = exact / attn_s / 1e12
    alg_tf = (exact + comp) / attn_s / 1e12
    # deepest global split level: groups must fit the LDS finisher
    fb = (136 * 1024) // (b * (d * es + 16))
    fb = min(fb, 1024 // b)
    F = 1
    while F * 2 <= fb:
        F *= 2
    rpt = 512 // (d // (16 // es))            # finisher rows per lane slot; 16 held per split
    while F > 1 and (F * b > 16 * rpt or ((F + 1) // 2) * b > 16 * (rpt // 2)):
        F //= 2
    lev, mx = 0, nb
    while mx > F:
        mx = (mx + 1) // 2
        lev += 1
    rb_bytes = reblock_bytes(H, N, d, b, es, lev, nb, 1 if args.layout == "q_reuse_k" else 2, Nv)
    rb_ms = st_mean[0] + st_mean[2]
    csrc = os.path.join(ROOT, "block_sparse_attention_mahalanobis_amd", "csrc")
    paired = not args.one_block and d == 128 and b == 128 and dtype == torch.bfloat16
    attn_kernel = "attn_pair_d128" if paired else "attn_mfma_d128"
    traffic = load_traffic("attn_full768_traffic.txt",
                           [os.path.join(csrc, f) for f in ("common.hpp", "k_attn.hip")],
                           "bytes_per_launch", attn_kernel) if args.config == "full768" and args.layout == "reblock" else None
    rb_traffic = load_traffic("reblock_full768_traffic.txt",
                              [os.path.join(csrc, f) for f in ("common.hpp", "k_whiten.hip", "k_split.hip",
                                                               "k_gather_summ.hip")],
                              "bytes_per_layer") if args.config == "full768" and args.layout == "reblock" else None

    base = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a sample (cpu_baseline)")
        base = cpu_baseline(w, topk, args.cpu_sample_blocks, ctx)
        log(f"cpu baseline {base['value']:.0f} ms projected ({base['sample']})")

    rec = {
        "metric": "Spark-Attn layer latency (ms) + exact-branch MFMA % peak, 245,952 tok @10% density",
        "value": round(layer_ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(layer_ms, 3),
        "wall_ms_per_step": round(wall_ms, 3),
        "step_ms_min_max": [round(float(per_step.min()), 3), round(float(per_step.max()), 3)],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded clustered Gaussian-mixture q/k on the latent grid, v ~ N(0,1))",
        "config": {"workload": w.name, "H": H, "N": N, "d": d, "block": b, "n_blocks": nb,
                   "topk": topk, "density": w.ratio, "layout": args.layout, "summary": "reweight",
                   **({"context_tokens": N - Nv, "context_blocks": nbt - nb} if ctx else {}),
                   **({"logits": "fp8 e4m3 (QK^T on fp8 MFMA, P V bf16)"} if args.fp8 else {})},
        "exact_mfma_pct_peak": round(100.0 * exact_tf / PEAK_BF16_TFLOPS, 2),
        "exact_mfma_pct_measured_peak": round(100.0 * exact_tf / peak_meas, 2),
        "stages_ms": {"reblock": round(st_mean[0], 3), "select": round(st_mean[1], 3),
                      "summarize": round(st_mean[2], 3), "attn": round(st_mean[3], 3)},
        "attn_tflops": {"exact": round(exact_tf, 1), "exact_plus_compressed": round(alg_tf, 1),
                        "exact_tflop": round(exact / 1e12, 2), "compressed_tflop": round(comp / 1e12, 2)},
        "reblock_summaries_hbm": {"algorithmic_gb": round(rb_bytes / 1e9, 1),
                                  "achieved_gbs": round(rb_bytes / (rb_ms * 1e-3) / 1e9, 1),
                                  "frac_of_8tbs": round(rb_bytes / (rb_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                                  "traffic_gb": None if rb_traffic is None else round(rb_traffic / 1e9, 1)},
        "roofline": {"kernel": attn_kernel + " (spark_attn)", "bound": "mfma",
                     "achieved": round(alg_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(alg_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "measured_peak": round(peak_meas, 1),
                     "measured_peak_note": "register-only v_mfma_f32_32x32x16_bf16 loop on this GPU "
                                           "(spark_mfma_peak_probe), best of 5 launches"},
        "cpu_baseline": base,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
