"""Parity at the full 768p layer shape -- 245,952 tokens (61 x 48 x 84 latent
grid), H = 40, d = 128, block 128, top-k ratio 0.1 -- in the launch
configuration that bench.py times (all 40 heads in one call of each entry
point, bf16).

* Stage injected.  For heads 0 and 39 the fp64 oracle computes the
  Spark-Reblock permutations, gathers and block means, block scores, the
  top-k routing, the Spark-Reweight summaries and, for sampled query blocks
  (the first two, the middle one, the last two -- the last is the 64-token
  ragged tail -- and three seeded random ones), the exact attention output.
  The GPU runs all 40 heads with those permutations, routing and summaries
  injected for the two heads (identity layout / its own routing for the
  others) and is compared: gathers bit for bit, block means and summaries
  within fp32 rounding, top-k bit for bit on the oracle's scores, sampled
  attention rows within the bf16 bar (rel-L2 <= 1e-2, max-abs <= 3e-2).
* End to end (the path bench.py times, no injection).  Properties that hold
  at any size: every head's two permutations are bijections of 0..N-1; each
  top-k row is strictly increasing, in range and of length k; under the
  kernel's own scores every selected block scores at least as high as every
  unselected one; all outputs are finite.  The kernel whitens in fp32 and
  stores the whitened vectors in bf16 for the split passes, so tokens whose
  split score lies within that rounding of a split threshold may land on the
  other side than in the fp64 oracle; the first two split levels of head 0
  must agree for all but 1% of the tokens (whitening by the wrong moment, or
  a wrong pole or score, moves about half of them).
* The splitter at full size, stage injected: the oracle's fp64 whitened
  queries and keys of head 0, rounded to bf16 (the splitter's storage
  precision), are split by the oracle and by the GPU; with equal inputs only
  fp32-vs-fp64 summation rounding can move a token, so the leaf (final
  128-token block) of all but a handful of tokens must agree.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS, make_head, round_to_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W = WORKLOADS["full768"]
B = W.block
CHECK_HEADS = (0, W.H - 1)


def say(msg):
    print(msg, flush=True)


def host(t):
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _oracle_head(h, topk, qblocks):
    """fp64 oracle for one head, attention only for the sampled query blocks
    (rows of the permuted order)."""
    q, k, v = (x.astype(np.float64) for x in make_head(W, h))
    N = q.shape[0]
    perm_q, perm_k = O.reblock_head(q, k, B)
    qp, qbar = O.gather_pool(q, perm_q, B)
    kp, kbar = O.gather_pool(k, perm_k, B)
    vp = v[perm_k]
    S = O.block_scores(qbar, kbar)
    idx = O.select_topk(S, topk)
    qhat = O.anchor_query(q, N)
    ks, vs, beta = O.reweight_summaries(kp, vp, qhat, B)
    op = O.sparse_attention(qp, kp, vp, idx, ks, vs, beta, B, qblocks=qblocks)
    return dict(perm_q=perm_q, perm_k=perm_k, qp=qp, kp=kp, vp=vp, qbar=qbar, kbar=kbar, S=S,
                idx=idx, qhat=qhat, ks=ks, vs=vs, beta=beta, op=op)


@pytest.fixture(scope="module")
def full():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    H, N, d = W.H, W.N, W.d
    nb = O.n_blocks(N, B)
    topk = O.topk_from_ratio(W.ratio, nb)
    rng = np.random.default_rng(20261203)
    qblocks = sorted({0, 1, nb // 2, nb - 2, nb - 1, *rng.choice(nb, 3, replace=False).tolist()})
    say(f"[full] generating H={H} N={N} d={d}; oracle heads {CHECK_HEADS}, q-blocks {qblocks}")
    dt = torch.bfloat16
    qkv = [torch.empty((H, N, d), dtype=dt, device=DEV) for _ in range(3)]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for h, arrs in enumerate(ex.map(lambda hh: make_head(W, hh), range(H))):
            for t, a in zip(qkv, arrs):
                t[h].copy_(torch.from_numpy(a).to(dt))
    torch.cuda.synchronize()
    orc = {h: _oracle_head(h, topk, qblocks) for h in CHECK_HEADS}
    say("[full] oracle done")
    return dict(q=qkv[0], k=qkv[1], v=qkv[2], N=N, nb=nb, topk=topk, qblocks=qblocks, orc=orc)


def _check_sampled_rows(out_h, o, qblocks, N, label):
    rows = np.concatenate([np.arange(A * B, min((A + 1) * B, N)) for A in qblocks])
    got = host(out_h[torch.from_numpy(o["perm_q"][rows]).to(DEV)])
    want = o["op"][rows]
    err, mab = rel_l2(got, want), float(np.abs(got - want).max())
    say(f"[full] {label}: {len(rows)} sampled rows rel_l2={err:.3e} max_abs={mab:.3e}")
    assert err <= 1e-2 and mab <= 3e-2


def test_full_size_stage_injected(full):
    q, k, v, N, nb, topk = full["q"], full["k"], full["v"], full["N"], full["nb"], full["topk"]
    H = q.shape[0]
    pq = torch.arange(N, dtype=torch.int32).repeat(H, 1)
    pk = pq.clone()
    for h, o in full["orc"].items():
        pq[h] = torch.from_numpy(o["perm_q"].astype(np.int32))
        pk[h] = torch.from_numpy(o["perm_k"].astype(np.int32))
    g = L.spark_reblock(q, k, v, B, layout="given", perm_q=pq, perm_k=pk)
    torch.cuda.synchronize()
    for h, o in full["orc"].items():
        say(f"[full] head {h}: gathers, block means")
        assert np.array_equal(host(g["q_p"][h])[:N], o["qp"])
        assert np.array_equal(host(g["k_p"][h])[:N], o["kp"])
        vp = host(g["v_pt"][h]).transpose(0, 2, 1).reshape(nb * B, -1)
        assert np.array_equal(vp[:N], o["vp"])
        assert np.all(vp[N:] == 0)
        np.testing.assert_allclose(host(g["qbar"][h]), o["qbar"], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(g["kbar"][h]), o["kbar"], rtol=1e-5, atol=1e-5)

    # top-k on the oracle's scores, bit for bit
    S32 = np.stack([full["orc"][h]["S"] for h in CHECK_HEADS]).astype(np.float32)
    idx_s = L.spark_select(None, None, topk, N, B, scores_in=torch.from_numpy(S32).to(DEV))
    torch.cuda.synchronize()
    for i, h in enumerate(CHECK_HEADS):
        assert np.array_equal(host(idx_s[i]), O.select_topk(S32[i].astype(np.float64), topk))

    # routing: the kernel's own for every head, the oracle's for the checked ones
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, B)
    anchor = g["anchor"].clone()
    for h, o in full["orc"].items():
        idx[h] = torch.from_numpy(o["idx"].astype(np.int32)).to(DEV)
        anchor[h] = torch.from_numpy(o["qhat"].astype(np.float32)).to(DEV)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], anchor, N, B)
    torch.cuda.synchronize()
    for h, o in full["orc"].items():
        say(f"[full] head {h}: summaries")
        np.testing.assert_allclose(host(ks[h]), o["ks"], rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(vs[h]), o["vs"], rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(bias[h]), o["beta"], rtol=2e-5, atol=2e-5)
        ks[h] = torch.from_numpy(o["ks"].astype(np.float32)).to(DEV)
        vs[h] = torch.from_numpy(o["vs"].astype(np.float32)).to(DEV)
        bias[h] = torch.from_numpy(o["beta"].astype(np.float32)).to(DEV)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, B, perm_q=g["perm_q"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    for h, o in full["orc"].items():
        _check_sampled_rows(out[h], o, full["qblocks"], N, f"head {h}")


def _group_labels(perm, N, nb, levels):
    """Group index (0 .. 2^levels - 1) of every token after the first
    `levels` capacity splits: the left child of a group of m blocks takes the
    first ceil(m/2) blocks of its slot range."""
    lab = np.zeros(N, np.int64)
    ranges = [(0, nb)]
    for _ in range(levels):
        nxt = []
        for s, m in ranges:
            nl = (m + 1) // 2
            nxt += [(s, nl), (s + nl, m - nl)]
        ranges = nxt
    for gi, (s, m) in enumerate(ranges):
        lo, hi = s * B, min((s + m) * B, N)
        lab[perm[lo:hi]] = gi
    return lab


def test_full_size_end_to_end_properties(full):
    q, k, v, N, nb, topk = full["q"], full["k"], full["v"], full["N"], full["nb"], full["topk"]
    H = q.shape[0]
    g = L.spark_reblock(q, k, v, B)
    idx, S = L.spark_select(g["qbar"], g["kbar"], topk, N, B, want_scores=True)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, B)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, B, perm_q=g["perm_q"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    # bijections, on the device
    ar = torch.arange(N, dtype=torch.int32, device=DEV)
    for name in ("perm_q", "perm_k"):
        srt = torch.sort(g[name].long(), dim=1).values.int()
        assert bool((srt == ar).all()), name
    # top-k rows: strictly increasing, in range
    assert int(idx.min()) >= 0 and int(idx.max()) < nb
    if topk > 1:
        assert bool((idx[:, :, 1:] > idx[:, :, :-1]).all())
    # selected blocks score at least as high as unselected ones (kernel scores)
    for h in CHECK_HEADS:
        Sh = S[h]
        sel = torch.zeros_like(Sh, dtype=torch.bool)
        sel.scatter_(1, idx[h].long(), True)
        worst_sel = torch.where(sel, Sh, torch.full_like(Sh, float("inf"))).min(dim=1).values
        best_uns = torch.where(sel, torch.full_like(Sh, -float("inf")), Sh).max(dim=1).values
        assert bool((worst_sel >= best_uns).all()), h
    # the first two split levels of head 0 against the oracle's fp64 split
    o = full["orc"][0]
    for name, ref in (("perm_q", o["perm_q"]), ("perm_k", o["perm_k"])):
        got = _group_labels(host(g[name][0]), N, nb, 2)
        want = _group_labels(ref, N, nb, 2)
        frac = float(np.mean(got != want))
        say(f"[full] head 0 {name}: {frac:.2e} of tokens in another level-2 group than the oracle's")
        assert frac <= 1e-2


def test_full_size_split_injected(full):
    N, nb = full["N"], full["nb"]
    q, k, _ = (x.astype(np.float64) for x in make_head(W, 0))
    xq = O.whiten(q, O.psd_sqrt(O.second_moment(k)))
    xk = O.whiten(k, O.psd_sqrt(O.second_moment(q)))
    x16 = np.stack([round_to_bf16(xq.astype(np.float32)), round_to_bf16(xk.astype(np.float32))])
    perm = host(L.spark_split(torch.from_numpy(x16).to(DEV).to(torch.bfloat16), B))
    torch.cuda.synchronize()
    for t, name in enumerate(("queries", "keys")):
        want = O.split_partition(x16[t].astype(np.float64), B)
        assert np.array_equal(np.sort(perm[t]), np.arange(N))
        leaf_g = np.empty(N, np.int64)
        leaf_g[perm[t]] = np.arange(N) // B
        leaf_o = np.empty(N, np.int64)
        leaf_o[want] = np.arange(N) // B
        moved = int(np.sum(leaf_g != leaf_o))
        say(f"[full] split of head 0 {name} (bf16 whitened input): {moved} of {N} tokens in another leaf")
        assert moved <= 64
