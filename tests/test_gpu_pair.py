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


@pytest.mark.parametrize("N,topk", [(100, 1), (200, 1), (200, 2), (300, 3)])
def test_pair_tiny_block_counts(N, topk):
    """n_b = 1 (a lone block, group 1 idle), 2 and 3, including full density."""
    want, outs = _run(N, topk, "random", seed=N + topk)
    assert rel_l2(outs[False], want) <= 1e-2 and np.abs(outs[False] - want).max() <= 3e-2
    assert rel_l2(outs[False], outs[True]) <= 5e-3


def test_large_block_count_falls_back_to_one_block():
    """n_b = 3,500 at 10%: the paired plan no longer fits in LDS, so the
    default takes the one-block kernel (bit-identical to SPARK_ATTN_ONE_BLOCK);
    sampled query blocks against the oracle."""
    rng = np.random.default_rng(21)
    N, d = 3500 * B - 17, 128
    nb = O.n_blocks(N, B)
    topk = O.topk_from_ratio(0.1, nb)
    q, k, v = (round_to_bf16(rng.standard_normal((N, d)).astype(np.float32)) for _ in range(3))
    idx = _routing("random", nb, topk, rng)[None]
    ks, vs, bias = O.reweight_summaries(k, v, O.anchor_query(q, N), B)
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)
    g = L.spark_reblock(t(q[None]), t(k[None]), t(v[None]), B, layout="identity")
    f = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)[None]).to(DEV)
    outs = [L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], torch.from_numpy(idx).to(DEV), f(ks), f(vs), f(bias),
                         N, B, perm_q=g["perm_q"], one_block=one) for one in (False, True)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    blocks = [0, 1, nb // 2, nb - 2, nb - 1]
    want = O.sparse_attention(q, k, v, idx[0], ks, vs, bias, B, qblocks=blocks)
    got = outs[0][0].float().cpu().numpy().astype(np.float64)
    rows = np.concatenate([np.arange(A * B, min(N, (A + 1) * B)) for A in blocks])
    e = rel_l2(got[rows], want[rows])
    say(f"[pair] fallback nb={nb}: sampled rel-L2 {e:.3e}")
    assert e <= 1e-2 and np.abs(got[rows] - want[rows]).max() <= 3e-2


@pytest.mark.parametrize("ratio", [0.1, 0.2])
def test_pair_at_the_768p_block_count(ratio):
    """n_b = 1922 at 10% and 20% (the largest slot tables the paired plan
    takes at this size): sampled query blocks against the oracle and the
    whole output against the one-block kernel."""
    rng = np.random.default_rng(int(ratio * 100))
    N, d = 245952, 128
    nb = O.n_blocks(N, B)
    topk = O.topk_from_ratio(ratio, nb)
    q, k, v = (round_to_bf16(rng.standard_normal((N, d)).astype(np.float32)) for _ in range(3))
    idx = _routing("random", nb, topk, rng)[None]
    ks, vs, bias = O.reweight_summaries(k, v, O.anchor_query(q, N), B)
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)
    g = L.spark_reblock(t(q[None]), t(k[None]), t(v[None]), B, layout="identity")
    f = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)[None]).to(DEV)
    outs = [L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], torch.from_numpy(idx).to(DEV), f(ks), f(vs), f(bias),
                         N, B, perm_q=g["perm_q"], one_block=one) for one in (False, True)]
    torch.cuda.synchronize()
    a0, a1 = (o[0].float().cpu().numpy().astype(np.float64) for o in outs)
    assert rel_l2(a0, a1) <= 5e-3
    blocks = [0, 1, 2, 3, nb // 2, nb // 2 + 1, nb - 2, nb - 1]
    want = O.sparse_attention(q, k, v, idx[0], ks, vs, bias, B, qblocks=blocks)
    rows = np.concatenate([np.arange(A * B, min(N, (A + 1) * B)) for A in blocks])
    e = rel_l2(a0[rows], want[rows])
    say(f"[pair] nb={nb} topk={topk}: sampled rel-L2 {e:.3e}, vs one-block {rel_l2(a0, a1):.3e}")
    assert e <= 1e-2 and np.abs(a0[rows] - want[rows]).max() <= 3e-2


@pytest.mark.parametrize("Nv,Nc,topk,kind", [(15900, 1000, 13, "random"), (15872, 2048, 7, "disjoint"),
                                              (9000, 100, 71, "identical")])
def test_pair_with_context_tokens(Nv, Nc, topk, kind):
    """SPARK_CONTEXT_EXACT: video query blocks run paired with every context
    tile shared by the pair (and the short last context block masked); the
    context query blocks run one per workgroup.  Video rows against the
    oracle's sparse attention with the context keys appended exactly,
    context rows against dense attention, and everything against the
    one-block kernel."""
    rng = np.random.default_rng(Nv + Nc + topk)
    N, d = Nv + Nc, 128
    q, k, v = (round_to_bf16(rng.standard_normal((N, d)).astype(np.float32) * s) for s in (1.5, 1.5, 1.0))
    nb = O.n_blocks(Nv, B)
    idx = _routing(kind, nb, topk, rng)[None]
    ks, vs, bias = O.reweight_summaries(k[:Nv], v[:Nv], O.anchor_query(q, Nv), B)
    want = np.concatenate([O.sparse_attention(q[:Nv], k[:Nv], v[:Nv], idx[0], ks, vs, bias, B,
                                              extra_k=k[Nv:], extra_v=v[Nv:]),
                           O.dense_attention(q[Nv:], k, v)])
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)
    g = L.spark_reblock(t(q[None]), t(k[None]), t(v[None]), B, layout="identity", n_anchor=Nv, context=True)
    f = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)[None]).to(DEV)
    outs = [L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], torch.from_numpy(idx).to(DEV), f(ks), f(vs), f(bias),
                         N, B, perm_q=g["perm_q"], n_anchor=Nv, context=True, one_block=one) for one in (False, True)]
    torch.cuda.synchronize()
    a0, a1 = (o[0].float().cpu().numpy().astype(np.float64) for o in outs)
    e, ev, ec = rel_l2(a0, want), rel_l2(a0[:Nv], want[:Nv]), rel_l2(a0[Nv:], want[Nv:])
    say(f"[pair] context Nv={Nv} Nc={Nc} topk={topk} {kind}: {e:.3e} (video {ev:.3e}, context {ec:.3e}), "
        f"vs one-block {rel_l2(a0, a1):.3e}")
    assert ev <= 1e-2 and ec <= 1e-2 and np.abs(a0 - want).max() <= 3e-2
    assert rel_l2(a0, a1) <= 5e-3


@pytest.mark.parametrize("kind", ["random", "disjoint", "identical"])
def test_pair_fp8_logits(kind):
    """SPARK_EXACT_FP8 on the paired schedule (E4M3 key tiles of 16 KB, the
    step's key scale from the plan): against the oracle's fp8 attention and
    the one-block fp8 kernel."""
    rng = np.random.default_rng(40 + len(kind))
    N, d, topk = 15900, 128, 13
    q, k, v = (round_to_bf16(rng.standard_normal((N, d)).astype(np.float32) * s) for s in (1.5, 1.5, 1.0))
    nb = O.n_blocks(N, B)
    idx = _routing(kind, nb, topk, rng)[None]
    ks, vs, bias = O.reweight_summaries(k, v, O.anchor_query(q, N), B)
    want = O.sparse_attention(q, k, v, idx[0], ks, vs, bias, B, fp8=True)
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)
    g = L.spark_reblock(t(q[None]), t(k[None]), t(v[None]), B, layout="identity")
    f = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)[None]).to(DEV)
    outs = [L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], torch.from_numpy(idx).to(DEV), f(ks), f(vs), f(bias),
                         N, B, perm_q=g["perm_q"], fp8=True, one_block=one) for one in (False, True)]
    torch.cuda.synchronize()
    a0, a1 = (o[0].float().cpu().numpy().astype(np.float64) for o in outs)
    e = rel_l2(a0, want)
    say(f"[pair] fp8 {kind}: {e:.3e}, vs one-block {rel_l2(a0, a1):.3e}")
    assert e <= 1e-2 and np.abs(a0 - want).max() <= 3e-2
    assert rel_l2(a0, a1) <= 5e-3
