"""GPU parity of the paired attention schedule (two adjacent query blocks
per workgroup, the key blocks both selected loaded once) against the fp64
oracle and against the one-block-per-workgroup kernel (SPARK_ATTN_ONE_BLOCK),
through the C ABI.

The routing is injected so that every branch of the pair plan runs: the two
blocks of a pair selecting disjoint sets (no shared tile), identical sets
(every tile shared), random sets (shared and own tiles, both parities of the
shared count), the last, partly padded block among the shared and among the
own tiles, an odd block count (the last pair has one block), top-1 and full
density.  Bars: bf16 attention rel-L2 <= 1e-2 and max-abs <= 3e-2 against
the oracle; the two schedules differ only in fp32 summation order, so
against each other rel-L2 <= 5e-3.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()


def say(msg):
    print(msg, flush=True)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _routing(kind, nb, topk, rng):
    """[nb, topk] strictly increasing block ids per query block."""
    rows = []
    for A in range(0, nb, 2):
        forced = nb - 1 if (A // 2) % 3 == 0 else None   # put the padded last block in now and then
        if kind == "identical":
            s = rng.choice(nb, topk, replace=False)
            if forced is not None and forced not in s:
                s[0] = forced
            pair = [s, s]
        elif kind == "disjoint":
            perm = rng.permutation(nb)
            if forced is not None:
                perm = np.concatenate([[forced], perm[perm != forced]])
                if (A // 2) % 2:     # the last block in the odd block's own list
                    perm = np.concatenate([perm[1:topk + 1], perm[:1], perm[topk + 1:]])
            pair = [perm[:topk], perm[topk:2 * topk]]
        else:   # random: independent draws
            pair = [rng.choice(nb, topk, replace=False) for _ in range(2)]
            if forced is not None:
                for s in pair:
                    if forced not in s:
                        s[-1] = forced
        rows += [np.sort(p) for p in pair]
    idx = np.stack(rows[:nb]).astype(np.int32)
    assert all(len(set(r)) == topk for r in idx)
    return idx


def _run(N, topk, kind, seed):
    rng = np.random.default_rng(seed)
    H, d = 1, 128
    q, k, v = (round_to_bf16(rng.standard_normal((H, N, d)).astype(np.float32) * s) for s in (1.5, 1.5, 1.0))
    nb = O.n_blocks(N, B)
    idx = np.stack([_routing(kind, nb, topk, rng) for _ in range(H)])
    want, sums = [], []
    for h in range(H):
        ks, vs, bias = O.reweight_summaries(k[h], v[h], O.anchor_query(q[h], N), B)
        sums.append((ks, vs, bias))
        want.append(O.sparse_attention(q[h], k[h], v[h], idx[h], ks, vs, bias, B))
    want = np.stack(want)
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)
    g = L.spark_reblock(t(q), t(k), t(v), B, layout="identity")
    f32 = lambda i: torch.from_numpy(np.stack([s[i] for s in sums]).astype(np.float32)).to(DEV)
    idx_d = torch.from_numpy(idx).to(DEV)
    outs = {}
    for one in (False, True):
        out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx_d, f32(0), f32(1), f32(2), N, B,
                           perm_q=g["perm_q"], one_block=one)
        torch.cuda.synchronize()
        outs[one] = out.float().cpu().numpy().astype(np.float64)
    return want, outs


@pytest.mark.parametrize("kind", ["random", "disjoint", "identical"])
@pytest.mark.parametrize("N,topk", [(16000, 13), (15900, 7), (9000, 1)])
def test_pair_schedule_matches_oracle_and_one_block(kind, N, topk):
    say(f"[pair] {kind} N={N} topk={topk}")
    want, outs = _run(N, topk, kind, seed=11 + N + topk)
    e_pair = rel_l2(outs[False], want)
    e_one = rel_l2(outs[True], want)
    e_pp = rel_l2(outs[False], outs[True])
    say(f"[pair] {kind} N={N} topk={topk}: pair {e_pair:.3e} one-block {e_one:.3e} between {e_pp:.3e}")
    assert e_pair <= 1e-2 and np.abs(outs[False] - want).max() <= 3e-2
    assert e_one <= 1e-2 and np.abs(outs[True] - want).max() <= 3e-2
    assert e_pp <= 5e-3


def test_pair_full_density_odd_block_count():
    """topk = n_b with an odd n_b: no compressed tiles, every tile shared,
    the last pair has one block."""
    N = 125 * 128 - 50
    nb = O.n_blocks(N, B)
    want, outs = _run(N, nb, "identical", seed=5)
    e = rel_l2(outs[False], want)
    say(f"[pair] full density nb={nb}: {e:.3e}")
    assert e <= 1e-2 and np.abs(outs[False] - want).max() <= 3e-2
    assert rel_l2(outs[False], outs[True]) <= 5e-3
