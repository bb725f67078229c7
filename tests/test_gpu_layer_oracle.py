"""End-to-end parity of the composed layer against the fp64 oracle, for the
layouts and inputs the other GPU tests check only through properties or
through the HIP path itself ("Spark-H3" blog, 01 / Method: Spark-Reblock:
the hierarchical partitioner and the BSA(Q_A) equation; comfyui-wiki news
item, "Workflows": reblock_layout=q_reuse_k; the blog's Spark-Ref2VA Preview
and 02 / Method: Spark-Reweight: the anchor is the mean of the video
queries).

* Reblock and q_reuse_k layers (draft 16x24x42 grid, bf16, a ragged
  16,100-token draft, and the tiny fp32 shapes; 10% and 20% density):
  spark_layer equals its four steps bit for bit, and its output equals, row
  by row, the oracle's layer run on the GPU's own permutations and routing
  (scores that select exactly the GPU's blocks) at the fp32 (rel-L2 <= 1e-5)
  or bf16 (rel-L2 <= 1e-2, max-abs <= 3e-2) bar.  The GPU's partition itself
  is compared with the oracle's fp64 partition: tokens of the first two split
  levels must agree for all but 1% (the split runs on bf16 / fp32 whitened
  vectors, so tokens within that rounding of a split threshold may move).
* Reference frames without the context flag (the 768p + 2-reference-frame
  layout in plain mode, here at draft size: the draft grid plus one 24x42
  reference frame, 20% density): every token is reblocked and attends
  sparsely; only the anchor is restricted to the video queries.  Stage
  injected against forward_head(n_anchor = video tokens): gathers and top-k
  bit for bit, anchor and summaries within fp32 rounding, attention at the
  bf16 bar; end to end on the GPU's own layout as above.
* i.i.d. N(0, 1) queries and keys (no spatio-temporal structure, the
  early-denoising regime of the Spark-Reblock noise paragraph): attention
  with the oracle's partition and routing injected at the bf16 bar, and the
  splitter on the oracle's whitened vectors rounded to bf16 leaf for leaf.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS, make_workload, round_to_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def say(msg):
    print(msg, flush=True)


def _tol(dt):
    return (1e-5, None) if dt == torch.float32 else (1e-2, 3e-2)


def _case(name):
    """q, k, v [H, N, d] float32, dtype, block"""
    if name == "tiny_f32":
        q, k, v = make_workload(WORKLOADS["tiny"])
        return q, k, v, torch.float32, 64
    if name == "tiny_f32_ragged":
        q, k, v = make_workload(WORKLOADS["tiny"])
        return q[:, :1000], k[:, :1000], v[:, :1000], torch.float32, 64
    if name == "draft_bf16":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[3, 17])
        return q, k, v, torch.bfloat16, 128
    if name == "draft_bf16_ragged":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[8])
        return q[:, :16100], k[:, :16100], v[:, :16100], torch.bfloat16, 128
    if name == "draft_iid":
        q, k, v = make_workload(WORKLOADS["sweep"].with_(iid=True), heads=[0, 5])
        return q, k, v, torch.bfloat16, 128
    raise KeyError(name)


def _group_labels(perm, N, nb, b, levels):
    """Group (0 .. 2^levels - 1) of every token after the first `levels`
    capacity splits: the left child of a group of m blocks takes the first
    ceil(m / 2) blocks of its slot range."""
    lab = np.zeros(N, np.int64)
    ranges = [(0, nb)]
    for _ in range(levels):
        nxt = []
        for s, m in ranges:
            nl = (m + 1) // 2
            nxt += [(s, nl), (s + nl, m - nl)] if m > 1 else [(s, m)]
        ranges = nxt
    for gi, (s, m) in enumerate(ranges):
        lo, hi = s * b, min((s + m) * b, N)
        lab[perm[lo:hi]] = gi
    return lab


def _onehot_scores(ix, nb):
    S = np.zeros((ix.shape[0], nb))
    np.put_along_axis(S, ix.astype(np.int64), 1.0, axis=1)
    return S


def _layer_vs_oracle(name, ratio, layout):
    q, k, v, dt, b = _case(name)
    H, N, d = q.shape
    nb = O.n_blocks(N, b)
    topk = O.topk_from_ratio(ratio, nb)
    say(f"[layer] {name} {layout} ratio {ratio}: H={H} N={N} topk={topk}/{nb}")
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    g = L.spark_reblock(qd, kd, vd, b, layout=layout)
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, b)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
    steps = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
    layer = L.spark_layer(qd, kd, vd, b, topk, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(steps, layer)
    pq, pk, ix = host(g["perm_q"]), host(g["perm_k"]), host(idx)
    got = host(layer)
    qh, kh, vh = host(qd), host(kd), host(vd)
    rl, ma = _tol(dt)
    for h in range(H):
        for p in (pq[h], pk[h]):
            assert np.array_equal(np.sort(p), np.arange(N))
        if layout == "q_reuse_k":
            assert np.array_equal(pq[h], pk[h])
        # the oracle's layer on the GPU's permutations and routing
        r = O.forward_head(qh[h], kh[h], vh[h], b, topk, layout="given", perm_q=pq[h], perm_k=pk[h],
                           scores_in=_onehot_scores(ix[h], nb))
        assert np.array_equal(r.idx, ix[h])
        err = rel_l2(got[h], r.out)
        mab = float(np.abs(got[h] - r.out).max())
        say(f"[layer] {name} {layout} head {h}: vs oracle on the GPU's layout rel_l2={err:.3e} max_abs={mab:.3e}")
        assert err <= rl
        if ma is not None:
            assert mab <= ma
        # the GPU's partition against the oracle's own fp64 partition
        if layout == "q_reuse_k":
            ref = {"perm_k": O.reblock_keys(qh[h], kh[h], b)}
        else:
            rq, rk = O.reblock_head(qh[h], kh[h], b)
            ref = {"perm_q": rq, "perm_k": rk}
        for side, want in ref.items():
            gp = pq[h] if side == "perm_q" else pk[h]
            frac = float(np.mean(_group_labels(gp, N, nb, b, 2) != _group_labels(want, N, nb, b, 2)))
            say(f"[layer] {name} {layout} head {h} {side}: {frac:.2e} of tokens in another level-2 group")
            assert frac <= 1e-2


@pytest.mark.parametrize("name,ratio", [("tiny_f32", 0.25), ("tiny_f32_ragged", 0.25),
                                        ("draft_bf16", 0.1), ("draft_bf16", 0.2),
                                        ("draft_bf16_ragged", 0.1), ("draft_bf16_ragged", 0.2)])
def test_reblock_layer_matches_oracle_on_gpu_layout(name, ratio):
    _layer_vs_oracle(name, ratio, "reblock")


@pytest.mark.parametrize("name,ratio", [("tiny_f32_ragged", 0.25), ("draft_bf16", 0.1),
                                        ("draft_bf16_ragged", 0.2)])
def test_q_reuse_k_layer_matches_oracle_on_gpu_layout(name, ratio):
    _layer_vs_oracle(name, ratio, "q_reuse_k")


# --- reference frames, plain mode (no context flag) --------------------------

REF_DRAFT = WORKLOADS["draft"].with_(ref_grid=(1, 24, 42), ref_components=8, ratio=0.2)


@pytest.fixture(scope="module")
def refcase():
    w = REF_DRAFT
    q, k, v = make_workload(w, heads=[2])
    N, nv, b = w.N, w.n_anchor, w.block
    nb = O.n_blocks(N, b)
    topk = O.topk_from_ratio(w.ratio, nb)
    say(f"[ref] N={N} video={nv} topk={topk}/{nb}")
    res = [O.forward_head(q[h], k[h], v[h], b, topk, n_anchor=nv) for h in range(q.shape[0])]
    return q, k, v, N, nv, b, nb, topk, res


def test_reference_frames_plain_stage_injected(refcase):
    q, k, v, N, nv, b, nb, topk, res = refcase
    dt = torch.bfloat16
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    g = L.spark_reblock(dev(q, dt), dev(k, dt), dev(v, dt), b, layout="given", perm_q=pq, perm_k=pk,
                        n_anchor=nv)
    S32 = np.stack([r.scores for r in res]).astype(np.float32)
    idx = L.spark_select(None, None, topk, N, b, scores_in=torch.from_numpy(S32).to(DEV))
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
    torch.cuda.synchronize()
    for h, r in enumerate(res):
        assert np.array_equal(host(g["q_p"][h])[:N], r.qp)
        assert np.array_equal(host(g["k_p"][h])[:N], r.kp)
        np.testing.assert_allclose(host(g["qbar"][h]), r.qbar, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(g["kbar"][h]), r.kbar, rtol=1e-5, atol=1e-5)
        # the anchor averages the video queries only
        np.testing.assert_allclose(host(g["anchor"][h]), r.anchor, rtol=1e-5, atol=1e-5)
        assert np.abs(host(g["anchor"][h]) - q[h].astype(np.float64).mean(axis=0)).max() > 1e-3
        assert np.array_equal(host(idx[h]), O.select_topk(S32[h].astype(np.float64), topk))
        np.testing.assert_allclose(host(ks[h]), r.ksum, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(vs[h]), r.vsum, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(bias[h]), r.bias, rtol=2e-5, atol=2e-5)
        got = host(out[h])
        err, mab = rel_l2(got, r.out), float(np.abs(got - r.out).max())
        say(f"[ref] head {h}: stage-injected attention rel_l2={err:.3e} max_abs={mab:.3e}")
        assert err <= 1e-2 and mab <= 3e-2


def test_reference_frames_plain_end_to_end(refcase):
    q, k, v, N, nv, b, nb, topk, res = refcase
    dt = torch.bfloat16
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    g = L.spark_reblock(qd, kd, vd, b, n_anchor=nv)
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, b)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
    steps = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
    layer = L.spark_layer(qd, kd, vd, b, topk, n_anchor=nv)
    torch.cuda.synchronize()
    assert torch.equal(steps, layer)
    pq, pk, ix, got = host(g["perm_q"]), host(g["perm_k"]), host(idx), host(layer)
    for h, r0 in enumerate(res):
        # every token, reference frames included, is reblocked
        for p in (pq[h], pk[h]):
            assert np.array_equal(np.sort(p), np.arange(N))
        r = O.forward_head(q[h], k[h], v[h], b, topk, n_anchor=nv, layout="given", perm_q=pq[h],
                           perm_k=pk[h], scores_in=_onehot_scores(ix[h], nb))
        err, mab = rel_l2(got[h], r.out), float(np.abs(got[h] - r.out).max())
        say(f"[ref] head {h}: layer vs oracle on the GPU's layout rel_l2={err:.3e} max_abs={mab:.3e}")
        assert err <= 1e-2 and mab <= 3e-2
        for side, want in (("perm_q", r0.perm_q), ("perm_k", r0.perm_k)):
            gp = pq[h] if side == "perm_q" else pk[h]
            frac = float(np.mean(_group_labels(gp, N, nb, b, 2) != _group_labels(want, N, nb, b, 2)))
            say(f"[ref] head {h} {side}: {frac:.2e} of tokens in another level-2 group")
            assert frac <= 1e-2


# --- i.i.d. queries and keys ---------------------------------------------------

@pytest.mark.parametrize("ratio", [0.1, 0.3])
def test_iid_attention_stage_injected(ratio):
    q, k, v, dt, b = _case("draft_iid")
    H, N, d = q.shape
    nb = O.n_blocks(N, b)
    topk = O.topk_from_ratio(ratio, nb)
    res = [O.forward_head(q[h], k[h], v[h], b, topk) for h in range(H)]
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    g = L.spark_reblock(dev(q, dt), dev(k, dt), dev(v, dt), b, layout="given", perm_q=pq, perm_k=pk)
    S32 = np.stack([r.scores for r in res]).astype(np.float32)
    idx = L.spark_select(None, None, topk, N, b, scores_in=torch.from_numpy(S32).to(DEV))
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
    torch.cuda.synchronize()
    for h, r in enumerate(res):
        assert np.array_equal(host(idx[h]), O.select_topk(S32[h].astype(np.float64), topk))
        np.testing.assert_allclose(host(ks[h]), r.ksum, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(bias[h]), r.bias, rtol=2e-5, atol=2e-5)
        got = host(out[h])
        err, mab = rel_l2(got, r.out), float(np.abs(got - r.out).max())
        say(f"[iid] ratio {ratio} head {h}: stage-injected attention rel_l2={err:.3e} max_abs={mab:.3e}")
        assert err <= 1e-2 and mab <= 3e-2


def test_iid_split_injected():
    q, k, _, _, b = _case("draft_iid")
    H, N, d = q.shape
    xs = []
    for h in range(H):
        qh, kh = q[h].astype(np.float64), k[h].astype(np.float64)
        xs.append(round_to_bf16(O.whiten(qh, O.psd_sqrt(O.second_moment(kh))).astype(np.float32)))
        xs.append(round_to_bf16(O.whiten(kh, O.psd_sqrt(O.second_moment(qh))).astype(np.float32)))
    x16 = np.stack(xs)
    perm = host(L.spark_split(torch.from_numpy(x16).to(DEV).to(torch.bfloat16), b))
    torch.cuda.synchronize()
    for t in range(x16.shape[0]):
        want = O.split_partition(x16[t].astype(np.float64), b)
        assert np.array_equal(np.sort(perm[t]), np.arange(N))
        leaf_g = np.empty(N, np.int64)
        leaf_g[perm[t]] = np.arange(N) // b
        leaf_o = np.empty(N, np.int64)
        leaf_o[want] = np.arange(N) // b
        moved = int(np.sum(leaf_g != leaf_o))
        say(f"[iid] split tree {t} (bf16 whitened input): {moved} of {N} tokens in another leaf")
        # equal inputs: only fp32-vs-fp64 summation rounding can move a token
        assert moved <= 16
