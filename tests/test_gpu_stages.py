"""GPU parity of every stage of the layer against the fp64 oracle, through
the C ABI, with the oracle's intermediates injected where an upstream
floating-point decision could legitimately differ (stage injection):

* gathers, top-k indices and the splitter on exact-arithmetic inputs are
  compared bit for bit;
* moments, square roots, whitening, block means, summaries and attention
  outputs within the tolerances of the fp32 / bf16 arithmetic:
  fp32 attention rel-L2 <= 1e-5; bf16 attention rel-L2 <= 1e-2 and
  max-abs <= 3e-2.
Sizes span several blocks and a ragged tail; every input is seeded.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS, make_head, make_workload, round_to_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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


# --------------------------------------------------------------------------
# cases: (name, q, k, v [H,N,d] float32 arrays, torch dtype, block, topk)
# --------------------------------------------------------------------------

def _case(name):
    if name == "tiny_f32":
        w = WORKLOADS["tiny"]
        q, k, v = make_workload(w)
        return q, k, v, torch.float32, 64, 4
    if name == "tiny_f32_ragged":        # N = 1000: last block of 40 tokens
        w = WORKLOADS["tiny"]
        q, k, v = make_workload(w)
        return q[:, :1000], k[:, :1000], v[:, :1000], torch.float32, 64, 4
    if name == "tiny_f32_tail1":         # N = 1025: a one-token tail block
        w = WORKLOADS["tiny"].with_(N_flat=1025)
        q, k, v = make_workload(w)
        return q, k, v, torch.float32, 64, 5
    if name == "tiny_bf16_b64":
        w = WORKLOADS["tiny"].with_(dtype="bf16")
        q, k, v = make_workload(w)
        return q, k, v, torch.bfloat16, 64, 4
    if name == "draft_bf16":             # 4 heads of the 16x24x42 latent
        q, k, v = make_workload(WORKLOADS["draft"], heads=[0, 1, 2, 3])
        return q, k, v, torch.bfloat16, 128, 13
    if name == "draft_bf16_ragged":      # N = 16100: last block of 100 tokens
        q, k, v = make_workload(WORKLOADS["draft"], heads=[5, 6])
        return q[:, :16100], k[:, :16100], v[:, :16100], torch.bfloat16, 128, 13
    if name == "draft_bf16_b32":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[7])
        return q[:, :4000], k[:, :4000], v[:, :4000], torch.bfloat16, 32, 13
    if name in ("draft_bf16_r20", "draft_bf16_r30"):   # the density sweep's 20% and 30%
        q, k, v = make_workload(WORKLOADS["draft"], heads=[9 if name.endswith("20") else 10])
        return q, k, v, torch.bfloat16, 128, O.topk_from_ratio(0.2 if name.endswith("20") else 0.3, 126)
    if name == "draft_bf16_b100":        # generic kernel (block not a multiple of 32)
        q, k, v = make_workload(WORKLOADS["draft"], heads=[8])
        return q[:, :3000], k[:, :3000], v[:, :3000], torch.bfloat16, 100, 4
    raise KeyError(name)


CASES = ["tiny_f32", "tiny_f32_ragged", "tiny_f32_tail1", "tiny_bf16_b64", "draft_bf16",
         "draft_bf16_ragged", "draft_bf16_b32", "draft_bf16_b100", "draft_bf16_r20", "draft_bf16_r30"]


@pytest.fixture(scope="module")
def oracle_runs():
    cache = {}

    def get(name):
        if name not in cache:
            q, k, v, dt, b, topk = _case(name)
            res = [O.forward_head(q[h], k[h], v[h], b, topk) for h in range(q.shape[0])]
            cache[name] = (q, k, v, dt, b, topk, res)
        return cache[name]
    return get


def _tol(dt):
    return (1e-5, None) if dt == torch.float32 else (1e-2, 3e-2)


@pytest.mark.parametrize("name", CASES)
def test_gather_pool_bit_exact_given_perm(name, oracle_runs):
    q, k, v, dt, b, topk, res = oracle_runs(name)
    H, N, d = q.shape
    say(f"[gather] {name} H={H} N={N} d={d} b={b}")
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    out = L.spark_reblock(dev(q, dt), dev(k, dt), dev(v, dt), b, layout="given", perm_q=pq, perm_k=pk)
    torch.cuda.synchronize()
    nb = O.n_blocks(N, b)
    for h in range(H):
        r = res[h]
        assert np.array_equal(host(out["q_p"][h])[:N], r.qp)
        assert np.all(host(out["q_p"][h])[N:] == 0)
        assert np.array_equal(host(out["k_p"][h])[:N], r.kp)
        vt = host(out["v_pt"][h])                       # [nb, d, b]
        vp = vt.transpose(0, 2, 1).reshape(nb * b, d)
        assert np.array_equal(vp[:N], r.vp)
        assert np.all(vp[N:] == 0)
        np.testing.assert_allclose(host(out["qbar"][h]), r.qbar, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(out["kbar"][h]), r.kbar, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(out["anchor"][h]), r.anchor, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name", CASES)
def test_summaries_match_oracle(name, oracle_runs):
    q, k, v, dt, b, topk, res = oracle_runs(name)
    H, N, d = q.shape
    say(f"[summaries] {name}")
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    g = L.spark_reblock(dev(q, dt), dev(k, dt), dev(v, dt), b, layout="given", perm_q=pq, perm_k=pk)
    anchor = torch.from_numpy(np.stack([r.anchor for r in res]).astype(np.float32)).to(DEV)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], anchor, N, b)
    torch.cuda.synchronize()
    for h in range(H):
        r = res[h]
        np.testing.assert_allclose(host(ks[h]), r.ksum, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(vs[h]), r.vsum, rtol=2e-5, atol=2e-5)
        np.testing.assert_allclose(host(bias[h]), r.bias, rtol=2e-5, atol=2e-5)
    if N % b == 1:      # one-token tail: bias 0, the summary is the token itself
        assert np.all(host(bias)[:, -1] == 0)
        assert np.array_equal(host(ks)[:, -1], np.stack([r.kp[-1] for r in res]))


@pytest.mark.parametrize("name", CASES)
def test_topk_bit_exact_on_given_scores(name, oracle_runs):
    q, k, v, dt, b, topk, res = oracle_runs(name)
    H, N, d = q.shape
    say(f"[select] {name}")
    S32 = np.stack([r.scores for r in res]).astype(np.float32)
    idx = L.spark_select(None, None, topk, N, b, scores_in=torch.from_numpy(S32).to(DEV))
    torch.cuda.synchronize()
    for h in range(H):
        want = O.select_topk(S32[h].astype(np.float64), topk)
        assert np.array_equal(host(idx[h]), want)


def test_topk_ties_nan_and_full_density():
    rng = np.random.default_rng(5)
    H, nb = 3, 300
    S = rng.integers(-4, 5, size=(H, nb, nb)).astype(np.float32)   # heavy ties
    S[0, 0, :] = 2.0
    S[1, 3, 10:20] = np.nan
    S[2, 7, :] = -np.inf
    S[2, 7, 5] = np.nan
    for topk in (1, 17, 150, 299, 300):
        idx = L.spark_select(None, None, topk, nb * 64, 64, scores_in=torch.from_numpy(S).to(DEV))
        torch.cuda.synchronize()
        got = host(idx)
        for h in range(H):
            want = O.select_topk(S[h].astype(np.float64), topk)
            assert np.array_equal(got[h], want), (h, topk)


@pytest.mark.parametrize("name", ["tiny_f32_ragged", "draft_bf16_ragged"])
def test_reblock_equals_its_stages(name):
    """spark_reblock equals its public stages composed: spark_moments, the
    two square roots (queries whitened by M_K^(1/2), keys by M_Q^(1/2)),
    spark_whiten and spark_split, permutations bit for bit."""
    q, k, v, dt, b, topk = _case(name)
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    g = L.spark_reblock(qd, kd, vd, b)
    MQ, MK, _ = L.spark_moments(qd, kd)
    pq = L.spark_split(L.spark_whiten(qd, L.spark_msqrt(MK)), b)
    pk = L.spark_split(L.spark_whiten(kd, L.spark_msqrt(MQ)), b)
    torch.cuda.synchronize()
    say(f"[stages] {name}: reblock vs composed stages")
    assert torch.equal(pq, g["perm_q"]) and torch.equal(pk, g["perm_k"])


def test_head_results_do_not_depend_on_the_head_batch():
    """Every step works per head and every launch plan depends on (N, d,
    block) only, so a head's layer output is the same whether it is
    processed alone, with one other head or with three.  N = 70,000: a plan
    that followed the head count would give 2 and 4 heads different moment
    chunks, hence different fp32 rounding."""
    rng = np.random.default_rng(11)
    H, N, d, b = 4, 70000, 128, 128
    q, k, v = (dev(rng.standard_normal((H, N, d)), torch.bfloat16) for _ in range(3))
    topk = L.topk_from_ratio(0.1, L.n_blocks(N, b))
    say(f"[batch] H={H} N={N} topk={topk}")
    full = L.spark_layer(q, k, v, b, topk)
    parts = [L.spark_layer(q[h0:h1].contiguous(), k[h0:h1].contiguous(), v[h0:h1].contiguous(), b, topk)
             for h0, h1 in ((0, 2), (2, 3), (3, 4))]
    torch.cuda.synchronize()
    assert torch.equal(full, torch.cat(parts))


@pytest.mark.parametrize("nb", [64, 65, 1922, 4096, 4097])
def test_topk_row_lengths(nb):
    """Rows of up to 4096 blocks keep their keys in registers, in slots of
    64; longer rows read them from LDS.  Both forms, at the slot boundaries,
    with ties and NaNs, select exactly what the oracle selects."""
    rng = np.random.default_rng(nb)
    S = rng.standard_normal((1, nb, nb)).astype(np.float32)
    S[0, :, ::7] = np.round(S[0, :, ::7])           # many equal scores
    S[0, 3, 10:20] = np.nan
    topk = max(1, nb // 10)
    say(f"[select] nb={nb} topk={topk}")
    got = host(L.spark_select(None, None, topk, nb, 1, scores_in=torch.from_numpy(S).to(DEV)))
    rows = sorted(set(range(min(nb, 24))) | set(range(max(0, nb - 24), nb))
                  | set(rng.integers(0, nb, 16).tolist()))
    for A in rows:
        want = O.select_topk(S[0, A:A + 1].astype(np.float64), topk)[0]
        assert np.array_equal(got[0, A], want), A


@pytest.mark.parametrize("nb,d", [(4097, 128), (3999, 64), (5000, 128)])
def test_topk_from_means_long_rows(nb, d):
    """Rows of more than 3968 blocks leave room for fewer than 8 query means
    per workgroup (7 at nb = 4097): the means then start at a 16-byte
    rounded offset after the score rows.  The scores the kernel computes
    from the means match the oracle's block scores, and its selection is
    exactly the oracle's selection on those scores."""
    rng = np.random.default_rng(nb + d)
    qbar = rng.standard_normal((1, nb, d)).astype(np.float32)
    kbar = rng.standard_normal((1, nb, d)).astype(np.float32)
    topk = max(1, nb // 10)
    say(f"[select] means nb={nb} d={d} topk={topk}")
    idx, S = L.spark_select(torch.from_numpy(qbar).to(DEV), torch.from_numpy(kbar).to(DEV), topk, nb, 1,
                            want_scores=True)
    torch.cuda.synchronize()
    S = host(S)[0]
    rows = sorted(set(range(16)) | set(range(nb - 16, nb)) | set(rng.integers(0, nb, 16).tolist()))
    want_S = O.block_scores(qbar[0].astype(np.float64)[rows], kbar[0].astype(np.float64))
    np.testing.assert_allclose(S[rows], want_S, rtol=1e-5, atol=1e-4)
    got = host(idx)[0]
    for A in rows:
        assert np.array_equal(got[A], O.select_topk(S[A:A + 1], topk)[0]), A


@pytest.mark.parametrize("name", ["tiny_f32", "draft_bf16"])
def test_scores_from_means_match_oracle(name, oracle_runs):
    q, k, v, dt, b, topk, res = oracle_runs(name)
    H, N, d = q.shape
    qbar = torch.from_numpy(np.stack([r.qbar for r in res]).astype(np.float32)).to(DEV)
    kbar = torch.from_numpy(np.stack([r.kbar for r in res]).astype(np.float32)).to(DEV)
    idx, S = L.spark_select(qbar, kbar, topk, N, b, want_scores=True)
    torch.cuda.synchronize()
    S = host(S)
    for h in range(H):
        np.testing.assert_allclose(S[h], res[h].scores, rtol=1e-5, atol=1e-4)
        # the selection is exact for the scores the kernel computed
        assert np.array_equal(host(idx[h]), O.select_topk(S[h], topk))


@pytest.mark.parametrize("name", CASES)
def test_attention_matches_oracle_with_injected_routing(name, oracle_runs):
    q, k, v, dt, b, topk, res = oracle_runs(name)
    H, N, d = q.shape
    say(f"[attn] {name}")
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    g = L.spark_reblock(dev(q, dt), dev(k, dt), dev(v, dt), b, layout="given", perm_q=pq, perm_k=pk)
    idx = torch.from_numpy(np.stack([r.idx for r in res]).astype(np.int32)).to(DEV)
    f32 = lambda a: torch.from_numpy(np.stack(a).astype(np.float32)).to(DEV)
    ks, vs, bias = f32([r.ksum for r in res]), f32([r.vsum for r in res]), f32([r.bias for r in res])
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
    torch.cuda.synchronize()
    got = host(out)
    want = np.stack([r.out for r in res])
    rl, ma = _tol(dt)
    err = rel_l2(got, want)
    say(f"[attn] {name} rel_l2={err:.3e} max_abs={np.abs(got - want).max():.3e}")
    assert err <= rl
    if ma is not None:
        assert np.abs(got - want).max() <= ma


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_full_density_equals_dense_attention(dt):
    """topk = n_b: no compressed branch; must equal dense softmax attention."""
    q, k, v = make_workload(WORKLOADS["draft"], heads=[9])
    N = 2000
    q, k, v = q[:, :N], k[:, :N], v[:, :N]
    b = 128
    nb = O.n_blocks(N, b)
    out = L.spark_layer(dev(q, dt), dev(k, dt), dev(v, dt), b, nb)
    torch.cuda.synchronize()
    want = O.dense_attention(q[0], k[0], v[0])
    got = host(out)[0]
    rl, ma = _tol(dt)
    assert rel_l2(got, want) <= rl
    if ma is not None:
        assert np.abs(got - want).max() <= ma


def test_block_size_one_equals_dense_attention():
    """block 1: every summary is its single token with zero bias, so the
    layer equals dense attention at any density."""
    rng = np.random.default_rng(3)
    N, d = 96, 64
    q, k, v = (rng.standard_normal((1, N, d)).astype(np.float32) for _ in range(3))
    for topk in (1, 7, 96):
        out = L.spark_layer(dev(q, torch.float32), dev(k, torch.float32), dev(v, torch.float32), 1, topk)
        torch.cuda.synchronize()
        assert rel_l2(host(out)[0], O.dense_attention(q[0], k[0], v[0])) <= 1e-5


# --------------------------------------------------------------------------
# reblock stages
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "draft_bf16_ragged"])
def test_moments_roots_whitening(name, oracle_runs):
    q, k, v, dt, b, topk, res = oracle_runs(name)
    H, N, d = q.shape
    say(f"[moments] {name}")
    MQ, MK, anchor = L.spark_moments(dev(q, dt), dev(k, dt))
    torch.cuda.synchronize()
    for h in range(H):
        np.testing.assert_allclose(host(MQ[h]), O.second_moment(q[h]), rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(MK[h]), O.second_moment(k[h]), rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(anchor[h]), O.anchor_query(q[h], N), rtol=1e-5, atol=1e-5)
    Ms = np.stack([O.second_moment(k[h]) for h in range(H)])
    W = L.spark_msqrt(torch.from_numpy(Ms.astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    for h in range(H):
        Wo = O.psd_sqrt(Ms[h])
        assert np.linalg.norm(host(W[h]) - Wo) / np.linalg.norm(Wo) < 2e-4
    Wt = torch.from_numpy(np.stack([O.psd_sqrt(Ms[h]) for h in range(H)]).astype(np.float32)).to(DEV)
    xh = L.spark_whiten(dev(q, dt), Wt)
    torch.cuda.synchronize()
    for h in range(H):
        want = O.whiten(q[h], O.psd_sqrt(Ms[h]))
        err = np.abs(host(xh[h]) - want).max()
        assert err < (1e-5 if dt == torch.float32 else 1.2e-2), err


def test_msqrt_edge_cases():
    d = 64
    M = np.zeros((3, d, d), dtype=np.float32)
    M[1] = np.diag(np.arange(d, dtype=np.float32))          # rank-deficient diagonal
    rng = np.random.default_rng(0)
    A = rng.standard_normal((d, 8)).astype(np.float32)
    M[2] = A @ A.T                                           # rank 8
    W = host(L.spark_msqrt(torch.from_numpy(M).to(DEV)))
    assert np.all(W[0] == 0)
    # the 1e-6 ridge of the iteration leaves sqrt(1e-6 ||M||_F) in null directions
    ridge = np.sqrt(1e-6 * np.linalg.norm(M[1]))
    np.testing.assert_allclose(np.diag(W[1])[1:], np.sqrt(np.arange(1, d)), atol=2e-3)
    assert abs(W[1][0, 0]) <= 1.5 * ridge
    off = W[1] - np.diag(np.diag(W[1]))
    assert np.abs(off).max() < 1e-4
    np.testing.assert_allclose(W[2] @ W[2], M[2], atol=2e-3 * np.abs(M[2]).max())


def _int_embed(rng, count, N, d, lo=-2, hi=2):
    return rng.integers(lo, hi + 1, size=(count, N, d)).astype(np.float32)


def test_split_hand_fixtures_exact():
    for fname in ("split_hand_example.json", "split_hand_example_odd.json"):
        g = json.load(open(os.path.join(GOLDEN, fname)))
        cases = g["cases"] if "cases" in g else [dict(block=g["block"], perm=g["perm"])]
        x2 = np.array(g["x"], dtype=np.float32)
        for case in cases:
            for dt, d in ((torch.float32, 64), (torch.bfloat16, 128)):
                x = np.zeros((1, x2.shape[0], d), dtype=np.float32)
                x[0, :, :2] = x2
                perm = L.spark_split(dev(x, dt), case["block"])
                torch.cuda.synchronize()
                assert host(perm)[0].tolist() == case["perm"], (fname, case["block"], dt)


@pytest.mark.parametrize("dt,N,d,b,count", [
    (torch.bfloat16, 4096, 128, 128, 3),     # global levels + LDS finisher
    (torch.bfloat16, 5000, 128, 128, 2),     # ragged: last block of 8 tokens
    (torch.float32, 3000, 64, 64, 2),
    (torch.bfloat16, 700, 64, 32, 2),
    (torch.float32, 257, 64, 1, 1),          # block 1: N leaves
    (torch.bfloat16, 2051, 128, 5, 2),       # odd N, block 5: group starts not 16-byte aligned
    (torch.bfloat16, 20000, 128, 128, 2),    # groups of > 64 blocks: the wide one-workgroup select
    (torch.bfloat16, 70000, 128, 128, 1),    # a group of > 512 blocks: the threshold by several workgroups
    (torch.float32, 20000, 64, 1, 2),        # six levels of > 512-block groups, 3 to 1 segments each
])
def test_split_bit_exact_on_integer_embeddings(dt, N, d, b, count):
    """Small-integer vectors: every sum and dot is exact in fp32, so the
    GPU partition must equal the oracle's bit for bit (ties included)."""
    rng = np.random.default_rng(N + d + b)
    x = _int_embed(rng, count, N, d)
    say(f"[split] N={N} d={d} b={b} count={count} {dt}")
    perm = host(L.spark_split(dev(x, dt), b))
    for t in range(count):
        want = O.split_partition(x[t].astype(np.float64), b)
        assert np.array_equal(perm[t], want), t


def test_split_all_ties():
    """Identical vectors everywhere: every decision is a tie -> identity."""
    x = np.ones((2, 2000, 64), dtype=np.float32)
    perm = host(L.spark_split(dev(x, torch.bfloat16), 64))
    assert np.array_equal(perm, np.tile(np.arange(2000), (2, 1)))
