"""fp64 CPU oracle of one Spark-Attn layer (Spark-Reblock, block top-k,
Spark-Reweight, fused exact + compressed attention).

TEST INFRASTRUCTURE ONLY.  This module exists to check the HIP library.
Only the test suite, the smoke check and the benchmark's ``cpu_baseline``
leg may import it; the product path never does, and it shares no code with
the HIP kernels or their binding.

Everything is plain NumPy in float64, one head at a time.  Inputs given in
bf16 or fp32 are upcast exactly.  Library primitives (matmul, eigh, sort)
serve as single steps; there is no blocking, fusion or reordering beyond
what each step below states.

Sources ("the pages"):
  [blog]  "Spark-H3: Adaptive Block Sparse Attention for MiniMax-H3",
          zechengtang.github.io/Spark-H3 -- sections "01 / Method:
          Spark-Reblock" (the d_Q equation, the hierarchical partitioner,
          the BSA equations for Q_A, K~_A, V~_A), "Discussion" (block-mean
          scoring, Top-K), "02 / Method: Spark-Reweight" (weighted
          summaries, log-mass bias, representative query, Jensen-gap
          figure).
  [readme] comfy.icu Spark-H3 package README, "Spark-Attn" section
          (reweighting gives different weights to tokens of each tail block).
  [news]  comfyui-wiki.com Spark-H3 news item, "What Spark-Attn changes"
          (the mean video query serves as one anchor per head),
          "Workflows" (the example workflows' reblock_layout=q_reuse_k).

Readings taken where the pages are silent:
  * split rule: two-pole capacity bisection (``split_group``);
  * binary splits, left child gets ceil(blocks/2) full blocks, so a short
    remainder block stays on the rightmost path and is the last leaf;
  * leaves in depth-first left-first order, ids ascending inside a leaf;
  * ties: lower original id (split) / lower block index (top-k) wins;
    NaN ranks last;
  * block score = q_bar_A . k_bar_B / sqrt(d), no bias;
  * top-k count = smallest count covering the ratio, in [1, n_blocks];
  * bias anchors the mean exponential of the block and the summary keeps
    the BSA multiplicity |B| (the all-ones vector in K~_A);
  * anchor = mean of the first ``n_anchor`` raw queries (video tokens);
  * moments are uncentred and use all N tokens;
  * fp8 mode (the Benchmark Results' FP8 runs; precision otherwise
    unstated): every attention logit q . k is taken from OCP E4M3 values --
    queries quantised per row, keys per block of b rows, summary keys per
    group of b consecutive blocks -- each group scaled by the smallest power
    of two that brings its largest magnitude to <= 448, rounded to nearest
    (ties to even); P and V stay in the bf16 path;
  * context mode ([blog] Spark-Reblock: context/sink tokens stay exact and
    lie outside the video-block Top-K budget): tokens [n_anchor, N) are
    context tokens.  Only the video tokens are partitioned, pooled, scored,
    selected and summarised; every video query also attends exactly to all
    context keys; a context query's row is exact dense attention over all
    N keys.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
tests/test_oracle_pins.py (closed forms, invariants, brute force, a
hand-derived partition fixture); none is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "n_blocks", "block_sizes", "topk_from_ratio", "second_moment", "psd_sqrt",
    "whiten", "argmin_lowest_id", "capacity_partition", "split_group", "split_partition", "reblock_head", "reblock_keys", "gather_pool",
    "block_scores", "select_topk", "anchor_query", "reweight_summaries",
    "mean_summaries", "sparse_attention", "dense_attention", "forward_head",
    "forward", "attention_mass_recall", "attention_mass_recall_rows", "log_mass_error",
    "log_mass_error_rows", "HeadResult",
    "E4M3_MAX", "e4m3_round", "pow2_scale", "quantize_e4m3_groups",
]


# ----------------------------------------------------------------------------
# Block bookkeeping
# ----------------------------------------------------------------------------

def n_blocks(N: int, b: int) -> int:
    """Blocks of ``b`` tokens covering N tokens; the last may be short."""
    return -(-N // b)


def block_sizes(N: int, b: int) -> np.ndarray:
    """Token count n_B of every block: b, ..., b, r with 1 <= r <= b."""
    nb = n_blocks(N, b)
    sz = np.full(nb, b, dtype=np.int64)
    sz[-1] = N - (nb - 1) * b
    return sz


def topk_from_ratio(ratio: float, nb: int) -> int:
    """Exact-branch budget: the blog's Top-K covers "the top 10% of video
    key-value blocks" (Spark-Reblock section); read as the smallest block
    count covering the ratio, clamped to [1, nb]."""
    return int(min(nb, max(1, math.ceil(ratio * nb - 1e-9))))


# ----------------------------------------------------------------------------
# Spark-Reblock ([blog] Spark-Reblock section, d_Q equation and partitioner)
# ----------------------------------------------------------------------------

def second_moment(x: np.ndarray) -> np.ndarray:
    """Uncentred second moment E[x x^T] over all rows of x [N, d]."""
    x = np.asarray(x, dtype=np.float64)
    return (x.T @ x) / x.shape[0]


def psd_sqrt(M: np.ndarray) -> np.ndarray:
    """Symmetric PSD square root M^{1/2}: eigendecomposition M = U L U^T,
    negative round-off eigenvalues clamped to 0, W = U sqrt(L) U^T."""
    M = np.asarray(M, dtype=np.float64)
    lam, U = np.linalg.eigh(0.5 * (M + M.T))
    lam = np.clip(lam, 0.0, None)
    return (U * np.sqrt(lam)) @ U.T


def whiten(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Unit-normalised whitened rows x^_i = W x_i / ||W x_i||, so that
    x^_i . x^_j = cos(W x_i, W x_j) and d_Q = 1 - x^_i . x^_j.
    A row whose whitened norm is 0 stays the zero vector."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    nrm = np.sqrt((y * y).sum(axis=1))
    out = np.zeros_like(y)
    nz = nrm > 0
    out[nz] = y[nz] / nrm[nz, None]
    return out


def argmin_lowest_id(vals: np.ndarray, ids: np.ndarray) -> int:
    """Index (into vals) of the minimum; ties -> lower id; NaN ranks last;
    -0 and +0 are equal values (the ids decide between them)."""
    vals = np.asarray(vals, dtype=np.float64) + 0.0   # folds -0 onto +0
    isn = np.isnan(vals)
    key = np.where(isn, 0.0, vals)
    order = np.lexsort((ids, key, isn))
    return int(order[0])


_argmin_lowest_id = argmin_lowest_id


def capacity_partition(s: np.ndarray, ids: np.ndarray, cap_left: int):
    """Left child = the cap_left members first in (s descending, id
    ascending) order, NaN scores last and -0 equal to +0; right child = the
    rest.  Both children are returned with ids ascending."""
    s = np.asarray(s, dtype=np.float64) + 0.0
    ids = np.asarray(ids)
    isn = np.isnan(s)
    key = np.where(isn, 0.0, -s)
    order = np.lexsort((ids, key, isn))
    return np.sort(ids[order[:cap_left]]), np.sort(ids[order[cap_left:]])


def split_group(xhat: np.ndarray, ids: np.ndarray, cap_left: int):
    """One capacity-constrained split of a group (ids ascending).

    The blog only says that each group is split "according to the
    corresponding distance while enforcing the assigned child capacities".
    Reading taken (two-pole capacity bisection):
      centroid      c   = sum_i x^_i
      pole A        = argmin_i x^_i . c      (farthest from the centroid)
      pole B        = argmin_i x^_i . x^_A   (farthest from A)
      score         s_i = x^_i . x^_A - x^_i . x^_B = d(i, B) - d(i, A)
      left child    = the cap_left members with the largest s (ties: lower
                      id; NaN last), right child = the rest.
    Both children are returned with ids ascending.
    """
    X = xhat[ids]
    c = X.sum(axis=0)
    a = argmin_lowest_id(X @ c, ids)
    xa = X[a]
    bi = argmin_lowest_id(X @ xa, ids)
    xb = X[bi]
    s = X @ xa - X @ xb
    return capacity_partition(s, ids, cap_left)


def split_partition(xhat: np.ndarray, b: int) -> np.ndarray:
    """Iterative hierarchical partitioner: start from all N ids as one group
    of n_blocks(N, b) blocks; level by level, every group with more than one
    block is split into a left child of ceil(blocks/2) full blocks and a
    right child with the rest, until every leaf is one block.  Returns
    perm [N] with perm[p] = original id at permuted position p (leaves in
    depth-first left-first order, ids ascending inside a leaf)."""
    N = xhat.shape[0]
    level = [np.arange(N, dtype=np.int64)]
    while True:
        nxt = []
        changed = False
        for g in level:
            nbg = n_blocks(g.shape[0], b)
            if nbg <= 1:
                nxt.append(g)
                continue
            cap_left = -(-nbg // 2) * b
            left, right = split_group(xhat, g, cap_left)
            nxt.extend([left, right])
            changed = True
        level = nxt
        if not changed:
            break
    return np.concatenate(level)


def reblock_head(q: np.ndarray, k: np.ndarray, b: int, n_split: Optional[int] = None):
    """Query and key permutations of one head.  Queries are whitened by
    M_K^{1/2} (keys' second moment), keys by M_Q^{1/2}: the opposite side's
    moment, as in the d_Q equation and its symmetric counterpart.  The
    moments use every row; only rows [0, n_split) (default: all) are
    partitioned -- the video tokens, when the rest are context tokens."""
    n = q.shape[0] if n_split is None else n_split
    MQ = second_moment(q)
    MK = second_moment(k)
    WQ = psd_sqrt(MK)
    WK = psd_sqrt(MQ)
    perm_q = split_partition(whiten(q[:n], WQ), b)
    perm_k = split_partition(whiten(k[:n], WK), b)
    return perm_q, perm_k


def reblock_keys(q: np.ndarray, k: np.ndarray, b: int, n_split: Optional[int] = None):
    """The key permutation alone (keys whitened by M_Q^{1/2}, split as in
    reblock_head).  The q_reuse_k layout ([news] Workflows: every example
    workflow of the release sets reblock_layout=q_reuse_k) groups the queries
    with this same key partition instead of splitting them separately."""
    n = k.shape[0] if n_split is None else n_split
    return split_partition(whiten(k[:n], psd_sqrt(second_moment(q))), b)


def gather_pool(x: np.ndarray, perm: np.ndarray, b: int):
    """Permuted rows x_p = x[perm] and their block means (over the real
    rows of each block, so the short last block divides by r)."""
    xp = np.asarray(x, dtype=np.float64)[perm]
    N = xp.shape[0]
    nb = n_blocks(N, b)
    means = np.zeros((nb, xp.shape[1]))
    for B in range(nb):
        means[B] = xp[B * b:min(N, (B + 1) * b)].mean(axis=0)
    return xp, means


# ----------------------------------------------------------------------------
# Block scoring and Top-K ([blog] Discussion: block-level means, fixed Top-K)
# ----------------------------------------------------------------------------

def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S[A, B] = q_bar_A . k_bar_B / sqrt(d)."""
    d = qbar.shape[1]
    return (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T) / math.sqrt(d)


def select_topk(S: np.ndarray, topk: int) -> np.ndarray:
    """Per row A the ``topk`` key blocks with the largest score (ties: lower
    block index; NaN ranks below -inf), returned in ascending block order."""
    nA, nB = S.shape
    idx = np.zeros((nA, topk), dtype=np.int64)
    cols = np.arange(nB)
    for A in range(nA):
        row = S[A]
        isn = np.isnan(row)
        key = np.where(isn, 0.0, -row)
        order = np.lexsort((cols, key, isn))
        idx[A] = np.sort(order[:topk])
    return idx


# ----------------------------------------------------------------------------
# Spark-Reweight ([blog] Spark-Reweight section; [readme]; [news])
# ----------------------------------------------------------------------------

def anchor_query(q: np.ndarray, n_anchor: int) -> np.ndarray:
    """Representative query: mean of the video queries (the first
    ``n_anchor`` rows in original order), one per head."""
    return np.asarray(q[:n_anchor], dtype=np.float64).mean(axis=0)


def reweight_summaries(kp: np.ndarray, vp: np.ndarray, qhat: np.ndarray, b: int):
    """Per key block B, scored once by the anchor q^:
        t_j   = q^ . k_j / sqrt(d)                (j in B)
        w_j   = exp(t_j) / sum_{j' in B} exp(t_j')
        k~_B  = sum_j w_j k_j,  v~_B = sum_j w_j v_j
        beta_B chosen so that exp(q^ . k~_B / sqrt(d) + beta_B) equals the
              block's mean exponential (1/n_B) sum_j exp(t_j), i.e.
        beta_B = log(sum_j exp(t_j)) - log(n_B) - q^ . k~_B / sqrt(d)
    (max-subtracted for range).  Returns k~ [nb, d], v~ [nb, d], beta [nb]."""
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    N, d = kp.shape
    nb = n_blocks(N, b)
    ks = np.zeros((nb, d))
    vs = np.zeros((nb, d))
    beta = np.zeros(nb)
    rs = 1.0 / math.sqrt(d)
    for B in range(nb):
        kB = kp[B * b:min(N, (B + 1) * b)]
        vB = vp[B * b:min(N, (B + 1) * b)]
        t = (kB @ qhat) * rs
        m = t.max()
        e = np.exp(t - m)
        Z = e.sum()
        w = e / Z
        ks[B] = w @ kB
        vs[B] = w @ vB
        beta[B] = m + math.log(Z) - math.log(kB.shape[0]) - float(qhat @ ks[B]) * rs
    return ks, vs, beta


def mean_summaries(kp: np.ndarray, vp: np.ndarray, b: int):
    """The BSA / Sol-Attn compressed branch: uniform block means k_bar,
    v_bar and no bias ([blog] Spark-Reblock section, K~_A / V~_A)."""
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    N, d = kp.shape
    nb = n_blocks(N, b)
    ks = np.zeros((nb, d))
    vs = np.zeros((nb, d))
    for B in range(nb):
        ks[B] = kp[B * b:min(N, (B + 1) * b)].mean(axis=0)
        vs[B] = vp[B * b:min(N, (B + 1) * b)].mean(axis=0)
    return ks, vs, np.zeros(nb)


# ----------------------------------------------------------------------------
# FP8 (OCP E4M3) logits ([blog] Benchmark Results: the DiT also runs in FP8)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0   # largest finite E4M3 magnitude: 1.75 * 2^8


def e4m3_round(x):
    """Round to the nearest OCP E4M3 value, ties to the even code: 3 mantissa
    bits, exponent bias 7, so normal numbers (|x| >= 2^-6) sit on a grid of
    2^(e-3) in the binade [2^e, 2^(e+1)) and subnormals on a grid of 2^-9.
    Inputs must satisfy |x| <= 448 (the callers scale them there)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_round: |x| > 448")
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 can misplace exact powers of two by one ulp: fix e so 2^e <= a < 2^(e+1)
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    quantum = np.where(a >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)
    return np.round(x / quantum) * quantum       # numpy rounds halves to even


def pow2_scale(amax):
    """Smallest power of two s with amax <= 448 s (1 for amax = 0): exact in
    any binary floating point, so every implementation picks the same s."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    e = math.frexp(amax)[1] - 9
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return 2.0 ** e


def quantize_e4m3_groups(x, group: int):
    """Rows of x in consecutive groups of ``group`` rows (the last may be
    short), each group scaled by pow2_scale of its largest magnitude and
    rounded to E4M3.  Returns (the dequantised rows, the per-group scales)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    n = x.shape[0]
    scales = np.zeros(max(1, -(-n // group)))
    for g0 in range(0, n, group):
        blk = x[g0:g0 + group]
        sc = pow2_scale(np.abs(blk).max() if blk.size else 0.0)
        scales[g0 // group] = sc
        out[g0:g0 + group] = e4m3_round(blk / sc) * sc
    return out, scales


# ----------------------------------------------------------------------------
# Two-branch attention ([blog] Spark-Reblock section, BSA(Q_A) equations)
# ----------------------------------------------------------------------------

def sparse_attention(qp, kp, vp, idx, ksum, vsum, bias, b: int, qblocks=None,
                     extra_k=None, extra_v=None, fp8: bool = False) -> np.ndarray:
    """BSA(Q_A) = Softmax(Q_A K~_A^T / sqrt(d)) V~_A with one row-wise softmax
    over the concatenation, per key block B, of
        B in S_A : the exact rows K_B, V_B;
        B not in S_A : the summary k~_B, v~_B repeated |B| times (the
                       all-ones vector), its logit shifted by beta_B;
    plus, when given, the rows of ``extra_k`` / ``extra_v`` exactly for
    every query block (context/sink tokens: exact, outside the Top-K budget).
    fp8: the logits use E4M3 queries (per row), keys (per block of b rows,
    context keys per block of b rows of their own) and summary keys (per b
    consecutive blocks); values and weights are unchanged.
    The |B| identical summary rows are carried as one row of weight |B|.
    Returns the output in permuted order [N, d].  ``qblocks`` (optional)
    restricts the work to those query blocks; other rows stay 0."""
    qp = np.asarray(qp, np.float64)
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    N, d = qp.shape
    nb = n_blocks(N, b)
    sizes = block_sizes(N, b).astype(np.float64)
    rs = 1.0 / math.sqrt(d)
    if extra_k is None:
        xk = np.zeros((0, d))
        xv = np.zeros((0, vp.shape[1]))
    else:
        xk = np.asarray(extra_k, np.float64)
        xv = np.asarray(extra_v, np.float64)
    if fp8:
        qp = quantize_e4m3_groups(qp, 1)[0]
        kp = quantize_e4m3_groups(kp, b)[0]
        ksum = quantize_e4m3_groups(ksum, b)[0]
        if xk.shape[0]:
            xk = quantize_e4m3_groups(xk, b)[0]
    out = np.zeros((N, d))
    for A in (range(nb) if qblocks is None else qblocks):
        rows = slice(A * b, min(N, (A + 1) * b))
        QA = qp[rows]
        sel = np.zeros(nb, dtype=bool)
        sel[np.asarray(idx[A], dtype=np.int64)] = True
        ex = np.concatenate([np.arange(B * b, min(N, (B + 1) * b)) for B in np.nonzero(sel)[0]])
        un = np.nonzero(~sel)[0]
        logits = np.concatenate([QA @ kp[ex].T * rs, QA @ xk.T * rs,
                                 QA @ ksum[un].T * rs + bias[un][None, :]], axis=1)
        weight = np.concatenate([np.ones(ex.shape[0] + xk.shape[0]), sizes[un]])
        vals = np.concatenate([vp[ex], xv, vsum[un]], axis=0)
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m) * weight[None, :]
        out[rows] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return out


def dense_attention(q, k, v) -> np.ndarray:
    """Softmax(q k^T / sqrt(d)) v, fp64, no mask."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = q @ k.T / math.sqrt(q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# One head / one layer
# ----------------------------------------------------------------------------

@dataclass
class HeadResult:
    perm_q: np.ndarray
    perm_k: np.ndarray
    qp: np.ndarray
    kp: np.ndarray
    vp: np.ndarray
    qbar: np.ndarray
    kbar: np.ndarray
    scores: np.ndarray
    idx: np.ndarray
    anchor: np.ndarray
    ksum: np.ndarray
    vsum: np.ndarray
    bias: np.ndarray
    out: np.ndarray       # original token order
    n_video: int = -1     # context mode: rows [n_video, N) are context tokens


def forward_head(q, k, v, b: int, topk: int, n_anchor: Optional[int] = None,
                 layout: str = "reblock", perm_q=None, perm_k=None,
                 summary: str = "reweight", scores_in=None,
                 context: bool = False, fp8: bool = False) -> HeadResult:
    """Reblock -> select -> summarise -> attend -> scatter, one head.
    layout: "reblock" (Spark-Reblock), "q_reuse_k" (the key partition reused
    for the queries), "identity" (consecutive blocks, the
    fixed-partition BSA baseline) or "given" (perm_q / perm_k supplied).
    summary: "reweight" (Spark-Reweight) or "mean" (BSA mean pooling).
    scores_in: optional block scores to select from instead of q_bar.k_bar.
    context: tokens [n_anchor, N) are context/sink tokens ([blog]
    Spark-Reblock: they stay exact, outside the video-block Top-K budget):
    blocks, scores, Top-K and summaries cover the video tokens only (topk
    counts video blocks), every video query attends exactly to all context
    keys, and each context query's row is dense attention over all N keys.
    The permutations then fix the context tokens (perm[p] = p, p >= n_anchor);
    qp / kp / vp and the block arrays hold the video tokens only.
    fp8: the attention logits come from E4M3 operands (see sparse_attention);
    a context query's dense row then uses E4M3 queries (per row) and keys
    (video keys per block of the permuted order, context keys per block of
    their own), like the video rows."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N = q.shape[0]
    n_anchor = N if n_anchor is None else n_anchor
    nv = n_anchor if context else N
    if layout == "reblock":
        perm_q, perm_k = reblock_head(q, k, b, n_split=nv)
    elif layout == "q_reuse_k":
        perm_k = reblock_keys(q, k, b, n_split=nv)
        perm_q = perm_k.copy()
    elif layout == "identity":
        perm_q = np.arange(nv)
        perm_k = np.arange(nv)
    elif layout == "given":
        perm_q = np.asarray(perm_q, np.int64)[:nv]
        perm_k = np.asarray(perm_k, np.int64)[:nv]
    else:
        raise ValueError(layout)
    qv, kv, vv = q[:nv], k[:nv], v[:nv]
    qp, qbar = gather_pool(qv, perm_q, b)
    kp, kbar = gather_pool(kv, perm_k, b)
    vp = vv[perm_k]
    S = block_scores(qbar, kbar) if scores_in is None else np.asarray(scores_in, np.float64)
    idx = select_topk(S, topk)
    qhat = anchor_query(q, n_anchor)
    if summary == "reweight":
        ks, vs, beta = reweight_summaries(kp, vp, qhat, b)
    elif summary == "mean":
        ks, vs, beta = mean_summaries(kp, vp, b)
    else:
        raise ValueError(summary)
    op = sparse_attention(qp, kp, vp, idx, ks, vs, beta, b,
                          extra_k=k[nv:] if nv < N else None, extra_v=v[nv:] if nv < N else None,
                          fp8=fp8)
    out = np.zeros((N, q.shape[1]))
    out[perm_q] = op
    if nv < N:
        if fp8:
            kq = np.concatenate([quantize_e4m3_groups(kp, b)[0], quantize_e4m3_groups(k[nv:], b)[0]])
            out[nv:] = dense_attention(quantize_e4m3_groups(q[nv:], 1)[0], kq,
                                       np.concatenate([vp, v[nv:]]))
        else:
            out[nv:] = dense_attention(q[nv:], k, v)
        tail = np.arange(nv, N)
        perm_q = np.concatenate([perm_q, tail])
        perm_k = np.concatenate([perm_k, tail])
    return HeadResult(perm_q, perm_k, qp, kp, vp, qbar, kbar, S, idx, qhat, ks, vs, beta, out,
                      nv if context else -1)


def forward(q, k, v, b: int, topk: int, n_anchor: Optional[int] = None, **kw):
    """Whole layer [H, N, d] -> output [H, N, d] (heads are independent)."""
    return np.stack([forward_head(q[h], k[h], v[h], b, topk, n_anchor, **kw).out
                     for h in range(q.shape[0])])


# ----------------------------------------------------------------------------
# Diagnostics ([blog] ablation tables: attention-mass recall, abs log-mass error)
# ----------------------------------------------------------------------------

def attention_mass_recall_rows(res: HeadResult, b: int) -> np.ndarray:
    """Per query row p of the permuted order: the dense attention
    probability (softmax over every key of the head) that falls on the exact
    keys of row p's query block's selected key blocks (plain layers only)."""
    if res.n_video >= 0:
        raise ValueError("diagnostics are defined for layers without context tokens")
    N, d = res.qp.shape
    nb = n_blocks(N, b)
    rec = np.zeros(N)
    for A in range(nb):
        rows = slice(A * b, min(N, (A + 1) * b))
        s = res.qp[rows] @ res.kp.T / math.sqrt(d)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        ex = np.concatenate([np.arange(B * b, min(N, (B + 1) * b)) for B in res.idx[A]])
        rec[rows] = p[:, ex].sum(axis=1)
    return rec


def attention_mass_recall(res: HeadResult, b: int) -> float:
    """Mean over the head's query rows of attention_mass_recall_rows."""
    return float(attention_mass_recall_rows(res, b).mean())


def log_mass_error_rows(res: HeadResult, b: int) -> np.ndarray:
    """Per query row p of the permuted order ([blog] Spark-Reweight, the
    log-mass error of its ablation table and the Jensen-gap figure):
        | log sum_{B not in S_A} sum_{j in B} exp(q_p . k_j / sqrt(d))
          - log sum_{B not in S_A} |B| exp(q_p . k~_B / sqrt(d) + beta_B) |
    where S_A is the selection of row p's query block and |B| the token count
    of block B (the multiplicity of the summary in the effective keys).  0 for
    rows whose block selects every key block (plain layers only)."""
    if res.n_video >= 0:
        raise ValueError("diagnostics are defined for layers without context tokens")
    N, d = res.qp.shape
    nb = n_blocks(N, b)
    sizes = block_sizes(N, b).astype(np.float64)
    rs = 1.0 / math.sqrt(d)
    err = np.zeros(N)

    def lse(z):
        m = z.max(axis=1)
        return m + np.log(np.exp(z - m[:, None]).sum(axis=1))

    for A in range(nb):
        rows = slice(A * b, min(N, (A + 1) * b))
        sel = np.zeros(nb, dtype=bool)
        sel[res.idx[A]] = True
        un = np.nonzero(~sel)[0]
        if un.size == 0:
            continue
        tok = np.concatenate([np.arange(B * b, min(N, (B + 1) * b)) for B in un])
        QA = res.qp[rows]
        exact = QA @ res.kp[tok].T * rs
        approx = QA @ res.ksum[un].T * rs + res.bias[un][None, :] + np.log(sizes[un])[None, :]
        err[rows] = np.abs(lse(exact) - lse(approx))
    return err


def log_mass_error(res: HeadResult, b: int) -> float:
    """Mean of log_mass_error_rows over the rows whose query block leaves at
    least one key block unselected (0 if none does)."""
    N = res.qp.shape[0]
    nb = n_blocks(N, b)
    has_tail = np.zeros(N, dtype=bool)
    for A in range(nb):
        has_tail[A * b:min(N, (A + 1) * b)] = len(set(np.asarray(res.idx[A]).tolist())) < nb
    rows = log_mass_error_rows(res, b)
    return float(rows[has_tail].mean()) if has_tail.any() else 0.0
