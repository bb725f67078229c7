"""GPU parity of the fused attention at the edges of its online softmax, for
the paired schedule and the one-block kernel, against the fp64 oracle.

Both kernels keep a lazy softmax reference per row: a tile's probabilities
are taken against the reference already held, and only when a half-row sum
exceeds 2^12 (or the row has seen no finite logit yet) is the exact tile
maximum taken and the output and sums rescaled.  The clustered and Gaussian
inputs of the other tests rarely leave that fast path after the first tile.
Here the routing and the keys are built so that it is left on purpose:

* rising logits: the selected blocks' logits climb by ~10 nats per block in
  the order the tiles are visited, with one jump of ~100 nats (past the
  fp32 range of exp2, so the fast path's sums overflow to inf);
* a first tile with no finite logit: every summary of compressed tile 0 is
  masked because all of its blocks are selected.

The method is [blog] "Spark-H3: Adaptive Block Sparse Attention for
MiniMax-H3", 01 / Method: Spark-Reblock (the BSA(Q_A) equation) and 02 /
Method: Spark-Reweight (the summary tokens); the online softmax is exact
whatever the reference, so the bars are the ordinary bf16 ones: rel-L2
<= 1e-2 and max-abs <= 3e-2.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import round_to_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B = 128
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()


def say(msg):
    print(msg, flush=True)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _attend(q, k, v, idx):
    """Oracle and both GPU schedules on one head with injected routing."""
    N = q.shape[0]
    ks, vs, bias = O.reweight_summaries(k, v, O.anchor_query(q, N), B)
    want = O.sparse_attention(q, k, v, idx, ks, vs, bias, B)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a[None], dtype=np.float32)).to(DEV).to(torch.bfloat16)
    g = L.spark_reblock(t(q), t(k), t(v), B, layout="identity")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a[None], dtype=np.float32)).to(DEV)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx[None], dtype=np.int32)).to(DEV)
    outs = {}
    for one in (False, True):
        out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx_d, f32(ks), f32(vs), f32(bias), N, B,
                           perm_q=g["perm_q"], one_block=one)
        torch.cuda.synchronize()
        outs[one] = out.float().cpu().numpy()[0].astype(np.float64)
    return want, outs


def _check(name, want, outs):
    assert np.isfinite(want).all()
    for one, got in outs.items():
        e, ma = rel_l2(got, want), float(np.abs(got - want).max())
        say(f"[extremes] {name} {'one-block' if one else 'paired'}: rel_l2={e:.3e} max_abs={ma:.2e}")
        assert np.isfinite(got).all()
        assert e <= 1e-2 and ma <= 3e-2


@pytest.mark.parametrize("N", [16 * B, 16 * B - 37])
def test_rising_logits_force_rescales(N):
    """Blocks 8..15 selected by every query block, visited in that order
    after the compressed tile of blocks 0..7; block B's logits sit near
    10 B nats (+100 from block 12 on: exp2 of the fast path overflows)."""
    rng = np.random.default_rng(N)
    nb = O.n_blocks(N, B)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    a = 16.0
    q = a * u + rng.standard_normal((N, D))
    lvl = 10.0 * np.arange(nb) + np.where(np.arange(nb) >= 12, 100.0, 0.0)   # nats
    g = lvl * np.sqrt(D) / a                                                  # key gain along u
    blk = np.minimum(np.arange(N) // B, nb - 1)
    k = g[blk][:, None] * u[None, :] + 0.5 * rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    q, k, v = (round_to_bf16(x.astype(np.float32)).astype(np.float64) for x in (q, k, v))
    idx = np.tile(np.arange(8, 16), (nb, 1))
    want, outs = _attend(q, k, v, idx)
    _check(f"rising N={N}", want, outs)


def test_first_compressed_tile_fully_masked():
    """200 blocks, top-130 = blocks 0..127 plus two more per query block:
    every summary of compressed tile 0 is masked, so each row's first tile
    holds no finite logit."""
    rng = np.random.default_rng(7)
    N = 200 * B - 100
    nb = O.n_blocks(N, B)
    q, k, v = (round_to_bf16((rng.standard_normal((N, D)) * s).astype(np.float32)).astype(np.float64)
               for s in (1.5, 1.5, 1.0))
    rows = []
    for A in range(nb):
        extra = np.sort(rng.choice(np.arange(128, nb), 2, replace=False))
        rows.append(np.concatenate([np.arange(128), extra]))
    idx = np.stack(rows)
    want, outs = _attend(q, k, v, idx)
    _check("tile 0 masked", want, outs)
