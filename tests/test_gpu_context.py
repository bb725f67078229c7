"""GPU parity of the context mode ("Spark-H3" blog, 01 / Method:
Spark-Reblock: context/sink tokens stay exact and lie outside the
video-block Top-K budget), through the C ABI, against the fp64 oracle's
``forward_head(..., context=True)``.  Tokens [n_anchor, N) are context
tokens; the cases cover every attention kernel (generic fp32, attn_mfma at
block 32 / 64, the d = 128 block-128 kernel) with ragged video and context
tails, a single context token, and a context shorter than one block.

* Stage injected (the oracle's video permutations given): gathers
  (video blocks, then the context blocks in original order) bit for bit,
  block means and summaries within fp32 rounding, top-k on the oracle's
  scores bit for bit, attention with the oracle's routing at the fp32
  (rel-L2 <= 1e-5) / bf16 (rel-L2 <= 1e-2, max-abs <= 3e-2) bars.
* Full density: every row (video rows with the context keys, context rows)
  equals dense attention over all N tokens.
* End to end with the GPU's own Spark-Reblock: context positions are fixed
  points of both permutations, the video part is a bijection, spark_layer
  equals the four steps composed, and the output equals the oracle's layer
  on the GPU's permutations and routing.
* With n_anchor = N the flag changes nothing (bit-identical layer).
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS, make_workload

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


# (name) -> q, k, v [H, N, d] float32, dtype, block, topk, n_video
def _case(name):
    if name == "tiny_f32":               # generic kernel; video tail 42, context tail 22
        q, k, v = make_workload(WORKLOADS["tiny"])
        return q, k, v, torch.float32, 64, 4, 874
    if name == "tiny_f32_ctx1":          # a single context token
        q, k, v = make_workload(WORKLOADS["tiny"])
        return q, k, v, torch.float32, 64, 3, 1023
    if name == "tiny_bf16_b32":          # attn_mfma<64, 32>; context shorter than a block
        q, k, v = make_workload(WORKLOADS["tiny"].with_(dtype="bf16"))
        return q, k, v, torch.bfloat16, 32, 5, 1000
    if name == "draft_bf16_b64":         # attn_mfma<128, 64>; tails 8 and 40
        q, k, v = make_workload(WORKLOADS["draft"], heads=[3])
        return q[:, :6000], k[:, :6000], v[:, :6000], torch.bfloat16, 64, 8, 5000
    if name == "draft_bf16_b128":        # attn_mfma_d128; tails 48 and 80, two heads
        q, k, v = make_workload(WORKLOADS["draft"], heads=[5, 6])
        return q, k, v, torch.bfloat16, 128, 11, 14000
    raise KeyError(name)


CASES = ["tiny_f32", "tiny_f32_ctx1", "tiny_bf16_b32", "draft_bf16_b64", "draft_bf16_b128"]
_cache = {}


def _oracle(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _cache:
        q, k, v, dt, b, topk, nv = _case(name)
        res = [O.forward_head(q[h], k[h], v[h], b, topk, n_anchor=nv, context=True, **kw)
               for h in range(q.shape[0])]
        _cache[key] = (q, k, v, dt, b, topk, nv, res)
    return _cache[key]


def _padded(x, nb, b):
    out = np.zeros((nb * b, x.shape[1]))
    out[:x.shape[0]] = x
    return out


@pytest.mark.parametrize("name", CASES)
def test_context_stages_with_oracle_injected(name):
    q, k, v, dt, b, topk, nv, res = _oracle(name)
    H, N, d = q.shape
    nbv, nbc = O.n_blocks(nv, b), O.n_blocks(N - nv, b)
    say(f"[context] {name}: N={N} video={nv} ({nbv} blocks) context={N - nv} ({nbc} blocks) topk={topk}")
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    g = L.spark_reblock(dev(q, dt), dev(k, dt), dev(v, dt), b, layout="given", perm_q=pq, perm_k=pk,
                        n_anchor=nv, context=True)
    torch.cuda.synchronize()
    # gathers: video blocks in the oracle's order, then the context tokens
    qd, kd, vd = (host(dev(x, dt)) for x in (q, k, v))   # inputs as the GPU holds them
    for h in range(H):
        want_q = np.concatenate([_padded(qd[h][res[h].perm_q[:nv]], nbv, b), _padded(qd[h][nv:], nbc, b)])
        want_k = np.concatenate([_padded(kd[h][res[h].perm_k[:nv]], nbv, b), _padded(kd[h][nv:], nbc, b)])
        want_v = np.concatenate([_padded(vd[h][res[h].perm_k[:nv]], nbv, b), _padded(vd[h][nv:], nbc, b)])
        assert np.array_equal(host(g["q_p"][h]), want_q)
        assert np.array_equal(host(g["k_p"][h]), want_k)
        vt = host(g["v_pt"][h]).transpose(0, 2, 1).reshape(-1, d)
        assert np.array_equal(vt, want_v)
        np.testing.assert_allclose(host(g["qbar"][h]), res[h].qbar, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(g["kbar"][h]), res[h].kbar, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(g["anchor"][h]), res[h].anchor, rtol=2e-5, atol=2e-5)
    # top-k on the oracle's scores: video blocks only
    S32 = np.stack([r.scores for r in res]).astype(np.float32)
    idx = L.spark_select(None, None, topk, N, b, scores_in=torch.from_numpy(S32).to(DEV),
                         n_anchor=nv, context=True)
    torch.cuda.synchronize()
    for h in range(H):
        assert np.array_equal(host(idx[h]), O.select_topk(S32[h].astype(np.float64), topk))
    # summaries of the video blocks
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b, n_anchor=nv, context=True)
    torch.cuda.synchronize()
    for h in range(H):
        np.testing.assert_allclose(host(ks[h]), res[h].ksum, rtol=1e-4, atol=1e-4)
        np.testing.assert_allclose(host(vs[h]), res[h].vsum, rtol=1e-4, atol=1e-4)
        np.testing.assert_allclose(host(bias[h]), res[h].bias, rtol=1e-4, atol=1e-4)
    # attention with the oracle's routing and summaries
    oidx = torch.from_numpy(np.stack([r.idx for r in res]).astype(np.int32)).to(DEV)
    f32 = lambda a: torch.from_numpy(np.stack(a).astype(np.float32)).to(DEV)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], oidx, f32([r.ksum for r in res]),
                       f32([r.vsum for r in res]), f32([r.bias for r in res]), N, b, perm_q=g["perm_q"],
                       n_anchor=nv, context=True)
    torch.cuda.synchronize()
    got, want = host(out), np.stack([r.out for r in res])
    rl, ma = _tol(dt)
    err_v, err_c = rel_l2(got[:, :nv], want[:, :nv]), rel_l2(got[:, nv:], want[:, nv:])
    say(f"[context] {name}: video rows rel_l2={err_v:.3e}, context rows rel_l2={err_c:.3e}, "
        f"max_abs={np.abs(got - want).max():.2e}")
    assert err_v <= rl and err_c <= rl
    if ma is not None:
        assert np.abs(got - want).max() <= ma
    # the permuted-order output (perm_q = NULL): the same rows, padded layout
    outp = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], oidx, f32([r.ksum for r in res]),
                        f32([r.vsum for r in res]), f32([r.bias for r in res]), N, b, n_anchor=nv,
                        context=True)
    torch.cuda.synchronize()
    op = host(outp)
    for h in range(H):
        assert np.array_equal(op[h][:nv], host(out[h])[res[h].perm_q[:nv]])
        assert np.array_equal(op[h][nbv * b:nbv * b + N - nv], host(out[h])[nv:])
        assert not op[h][nv:nbv * b].any() and not op[h][nbv * b + N - nv:].any()


@pytest.mark.parametrize("name", ["tiny_f32", "draft_bf16_b64", "draft_bf16_b128"])
def test_context_full_density_equals_dense(name):
    q, k, v, dt, b, _, nv = _case(name)
    H, N, d = q.shape
    nbv = O.n_blocks(nv, b)
    out = L.spark_layer(dev(q, dt), dev(k, dt), dev(v, dt), b, nbv, n_anchor=nv, context=True)
    torch.cuda.synchronize()
    qd, kd, vd = (host(dev(x, dt)) for x in (q, k, v))
    want = np.stack([O.dense_attention(qd[h], kd[h], vd[h]) for h in range(H)])
    got = host(out)
    rl, ma = _tol(dt)
    err = rel_l2(got, want)
    say(f"[context] {name}: full density vs dense rel_l2={err:.3e}")
    assert err <= rl
    if ma is not None:
        assert np.abs(got - want).max() <= ma


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_bf16_b32", "draft_bf16_b128"])
def test_context_layer_end_to_end(name):
    q, k, v, dt, b, topk, nv = _case(name)
    H, N, d = q.shape
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    g = L.spark_reblock(qd, kd, vd, b, n_anchor=nv, context=True)
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, b, n_anchor=nv, context=True)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b, n_anchor=nv, context=True)
    steps = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"],
                         n_anchor=nv, context=True)
    layer = L.spark_layer(qd, kd, vd, b, topk, n_anchor=nv, context=True)
    torch.cuda.synchronize()
    assert torch.equal(steps, layer)
    pq, pk, ix = host(g["perm_q"]), host(g["perm_k"]), host(idx)
    tail = np.arange(nv, N)
    for h in range(H):
        for p in (pq[h], pk[h]):
            assert np.array_equal(np.sort(p[:nv]), np.arange(nv))
            assert np.array_equal(p[nv:], tail)
    # the oracle's layer on the GPU's permutations and routing (scores that
    # select exactly the GPU's blocks)
    qh, kh, vh = host(qd), host(kd), host(vd)
    nbv = O.n_blocks(nv, b)
    got = host(layer)
    rl, ma = _tol(dt)
    for h in range(H):
        S = np.zeros((nbv, nbv))
        np.put_along_axis(S, ix[h].astype(np.int64), 1.0, axis=1)
        r = O.forward_head(qh[h], kh[h], vh[h], b, topk, n_anchor=nv, layout="given", perm_q=pq[h],
                           perm_k=pk[h], scores_in=S, context=True)
        assert np.array_equal(r.idx, ix[h])
        err = rel_l2(got[h], r.out)
        say(f"[context] {name} head {h}: layer vs oracle on the GPU's layout rel_l2={err:.3e}")
        assert err <= rl
        if ma is not None:
            assert np.abs(got[h] - r.out).max() <= ma


def test_context_flag_without_context_tokens_changes_nothing():
    q, k, v, dt, b, topk, _ = _case("draft_bf16_b128")
    H, N, d = q.shape
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    a = L.spark_layer(qd, kd, vd, b, topk, n_anchor=N, context=True)
    c = L.spark_layer(qd, kd, vd, b, topk, n_anchor=N)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
