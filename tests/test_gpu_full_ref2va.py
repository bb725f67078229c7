"""Parity at the full reference-conditioned shape with context tokens exact:
245,952 video tokens plus two 48x84 reference frames (8,064 context tokens,
254,016 in all), H = 40, d = 128, block 128, top-k ratio 0.2 of the 1922
video blocks, all 40 heads in one call of each entry point (bf16).

Stage injected for head 0: the fp64 oracle computes the video permutations,
gathers and block means, scores, top-k, the Spark-Reweight summaries (anchor
over the video queries) and, for sampled rows, the exact output.  Checked:
gathers bit for bit (the video blocks in the oracle's order, then the
context tokens in their own blocks); top-k on the oracle's scores bit for
bit; block means and summaries within fp32 rounding; the video rows of the
first, middle and last query blocks and three seeded random ones (each also
attends every context key exactly) and 256 context rows (the first and last
128, each a dense row over all 254,016 keys) within the bf16 bar (rel-L2 <=
1e-2, max-abs <= 3e-2).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS, make_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W = WORKLOADS["ref2va"]
B = W.block


def say(msg):
    print(msg, flush=True)


def host(t):
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.fixture(scope="module")
def ref2va():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    H, N, d, nv = W.H, W.N, W.d, W.n_anchor
    nbv = O.n_blocks(nv, B)
    topk = O.topk_from_ratio(W.ratio, nbv)
    rng = np.random.default_rng(20261204)
    qblocks = sorted({0, nbv // 2, nbv - 1, *rng.choice(nbv, 3, replace=False).tolist()})
    say(f"[ref2va] generating H={H} N={N} (video {nv}) d={d}; topk={topk}; q-blocks {qblocks}")
    dt = torch.bfloat16
    qkv = [torch.empty((H, N, d), dtype=dt, device=DEV) for _ in range(3)]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for h, arrs in enumerate(ex.map(lambda hh: make_head(W, hh), range(H))):
            for t, a in zip(qkv, arrs):
                t[h].copy_(torch.from_numpy(a).to(dt))
    torch.cuda.synchronize()
    q, k, v = (x.astype(np.float64) for x in make_head(W, 0))   # bf16-exact values
    perm_q, perm_k = O.reblock_head(q, k, B, n_split=nv)
    qp, qbar = O.gather_pool(q[:nv], perm_q, B)
    kp, kbar = O.gather_pool(k[:nv], perm_k, B)
    vp = v[:nv][perm_k]
    S = O.block_scores(qbar, kbar)
    idx = O.select_topk(S, topk)
    qhat = O.anchor_query(q, nv)
    ks, vs, beta = O.reweight_summaries(kp, vp, qhat, B)
    op = O.sparse_attention(qp, kp, vp, idx, ks, vs, beta, B, qblocks=qblocks, extra_k=k[nv:], extra_v=v[nv:])
    crow = np.r_[nv:nv + 128, N - 128:N]
    oc = O.dense_attention(q[crow], k, v)
    say("[ref2va] oracle done")
    return dict(q=qkv[0], k=qkv[1], v=qkv[2], N=N, nv=nv, nbv=nbv, topk=topk, qblocks=qblocks, x=(q, k, v),
                perm_q=perm_q, perm_k=perm_k, qp=qp, kp=kp, vp=vp, qbar=qbar, kbar=kbar, S=S, idx=idx,
                qhat=qhat, ks=ks, vs=vs, beta=beta, op=op, crow=crow, oc=oc)


def test_ref2va_full_size_stage_injected(ref2va):
    r = ref2va
    q, k, v, N, nv, nbv, topk = r["q"], r["k"], r["v"], r["N"], r["nv"], r["nbv"], r["topk"]
    H, _, d = q.shape
    nbc = O.n_blocks(N - nv, B)
    pq = torch.arange(N, dtype=torch.int32).repeat(H, 1)
    pk = pq.clone()
    pq[0, :nv] = torch.from_numpy(r["perm_q"].astype(np.int32))
    pk[0, :nv] = torch.from_numpy(r["perm_k"].astype(np.int32))
    g = L.spark_reblock(q, k, v, B, layout="given", perm_q=pq, perm_k=pk, n_anchor=nv, context=True)
    torch.cuda.synchronize()
    say("[ref2va] head 0: gathers, block means")
    x_q, x_k, x_v = r["x"]
    for name, got, video, ctx in (("q_p", g["q_p"][0], r["qp"], x_q[nv:]), ("k_p", g["k_p"][0], r["kp"], x_k[nv:])):
        h0 = host(got)
        assert np.array_equal(h0[:nv], video), name
        assert not h0[nv:nbv * B].any(), name
        assert np.array_equal(h0[nbv * B:nbv * B + N - nv], ctx), name
        assert not h0[nbv * B + N - nv:].any(), name
    vt = host(g["v_pt"][0]).transpose(0, 2, 1).reshape(-1, d)
    assert np.array_equal(vt[:nv], r["vp"])
    assert np.array_equal(vt[nbv * B:nbv * B + N - nv], x_v[nv:])
    assert vt.shape[0] == (nbv + nbc) * B
    np.testing.assert_allclose(host(g["qbar"][0]), r["qbar"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(host(g["kbar"][0]), r["kbar"], rtol=1e-5, atol=1e-5)

    # top-k of the video blocks on the oracle's scores, bit for bit
    S32 = r["S"][None].astype(np.float32)
    idx_s = L.spark_select(None, None, topk, N, B, scores_in=torch.from_numpy(S32).to(DEV), n_anchor=nv,
                           context=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx_s[0]), O.select_topk(S32[0].astype(np.float64), topk))

    # routing and anchor: the kernel's for every head, the oracle's for head 0
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, B, n_anchor=nv, context=True)
    idx[0] = torch.from_numpy(r["idx"].astype(np.int32)).to(DEV)
    anchor = g["anchor"].clone()
    anchor[0] = torch.from_numpy(r["qhat"].astype(np.float32)).to(DEV)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], anchor, N, B, n_anchor=nv, context=True)
    torch.cuda.synchronize()
    say("[ref2va] head 0: summaries")
    np.testing.assert_allclose(host(ks[0]), r["ks"], rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(host(vs[0]), r["vs"], rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(host(bias[0]), r["beta"], rtol=2e-5, atol=2e-5)
    ks[0] = torch.from_numpy(r["ks"].astype(np.float32)).to(DEV)
    vs[0] = torch.from_numpy(r["vs"].astype(np.float32)).to(DEV)
    bias[0] = torch.from_numpy(r["beta"].astype(np.float32)).to(DEV)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, B, perm_q=g["perm_q"],
                       n_anchor=nv, context=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows = np.concatenate([np.arange(A * B, min((A + 1) * B, nv)) for A in r["qblocks"]])
    got = host(out[0][torch.from_numpy(r["perm_q"][rows]).to(DEV)])
    want = r["op"][rows]
    err, mab = rel_l2(got, want), float(np.abs(got - want).max())
    say(f"[ref2va] head 0: {len(rows)} sampled video rows rel_l2={err:.3e} max_abs={mab:.3e}")
    assert err <= 1e-2 and mab <= 3e-2
    gc = host(out[0][torch.from_numpy(r["crow"]).to(DEV)])
    err_c, mab_c = rel_l2(gc, r["oc"]), float(np.abs(gc - r["oc"]).max())
    say(f"[ref2va] head 0: {len(r['crow'])} context rows rel_l2={err_c:.3e} max_abs={mab_c:.3e}")
    assert err_c <= 1e-2 and mab_c <= 3e-2
