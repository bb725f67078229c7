"""GPU parity of the fp8 logits (SPARK_EXACT_FP8; the "Spark-H3" blog's
Benchmark Results run the DiT in FP8), through the C ABI, against the fp64
oracle's fp8 mode:

* spark_quant_e4m3 -- the quantisation the attention applies to key tiles,
  summary tiles and (in registers, by the same rule) query rows -- equals
  the oracle's quantize_e4m3_groups bit for bit: the same power-of-two
  scales and the same E4M3 values (decoded here from the format's
  definition), for bf16 and fp32 rows, groups of 1 and of a block, a
  ragged last group and an all-zero group.
* Attention with the oracle's routing and summaries injected, E4M3 logits,
  against the oracle's fp8 layer (the same E4M3 operands in fp64): the
  bf16 bars (rel-L2 <= 1e-2, max-abs <= 3e-2), since once both sides round
  the same operands what remains is the bf16 P and fp32 accumulation.
  Covered: the draft workload, a ragged tail, and context tokens.
* spark_layer in fp8 mode equals the four steps composed.
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


def e4m3_decode(codes):
    """Value of each OCP E4M3 code (sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent 0 subnormal; 0x7f / 0xff NaN)."""
    c = codes.astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


@pytest.mark.parametrize("dt,rows,group,d", [(torch.bfloat16, 1000, 128, 128), (torch.bfloat16, 257, 1, 128),
                                             (torch.float32, 300, 64, 64)])
def test_quantisation_bit_exact(dt, rows, group, d):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((rows, d)) * np.exp2(rng.integers(-20, 12, (rows, 1)))
    x[group:2 * group] = 0.0                      # an all-zero group (scale 1)
    xd = dev(x, dt)
    x8, sc = L.spark_quant_e4m3(xd, group)
    torch.cuda.synchronize()
    want, want_sc = O.quantize_e4m3_groups(host(xd), group)
    got_sc = host(sc)
    np.testing.assert_array_equal(got_sc, want_sc)
    deq = e4m3_decode(x8.cpu().numpy()) * np.repeat(got_sc, group)[:rows, None]
    np.testing.assert_array_equal(deq, want)
    say(f"[fp8] quantisation {dt} rows={rows} group={group}: bit-exact, scales 2^{int(np.log2(got_sc.min()))}"
        f"..2^{int(np.log2(got_sc.max()))}")


def _case(name):
    if name == "draft":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[0, 1])
        return q, k, v, 128, 13, None
    if name == "draft_ragged":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[5])
        return q[:, :16100], k[:, :16100], v[:, :16100], 128, 13, None
    if name == "draft_context":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[6])
        return q, k, v, 128, 11, 14000
    raise KeyError(name)


@pytest.mark.parametrize("name", ["draft", "draft_ragged", "draft_context"])
def test_fp8_attention_matches_oracle(name):
    q, k, v, b, topk, nv = _case(name)
    H, N, d = q.shape
    ctx = nv is not None
    dt = torch.bfloat16
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    qh, kh, vh = host(qd), host(kd), host(vd)     # the bf16 inputs, as both sides see them
    res = [O.forward_head(qh[h], kh[h], vh[h], b, topk, n_anchor=nv, context=ctx, fp8=True) for h in range(H)]
    pq = torch.from_numpy(np.stack([r.perm_q for r in res]).astype(np.int32))
    pk = torch.from_numpy(np.stack([r.perm_k for r in res]).astype(np.int32))
    g = L.spark_reblock(qd, kd, vd, b, layout="given", perm_q=pq, perm_k=pk, n_anchor=nv, context=ctx)
    idx = torch.from_numpy(np.stack([r.idx for r in res]).astype(np.int32)).to(DEV)
    f32 = lambda a: torch.from_numpy(np.stack(a).astype(np.float32)).to(DEV)
    out = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, f32([r.ksum for r in res]), f32([r.vsum for r in res]),
                       f32([r.bias for r in res]), N, b, perm_q=g["perm_q"], n_anchor=nv, context=ctx, fp8=True)
    torch.cuda.synchronize()
    got, want = host(out), np.stack([r.out for r in res])
    err, mab = rel_l2(got, want), float(np.abs(got - want).max())
    plain = np.stack([O.forward_head(qh[h], kh[h], vh[h], b, topk, n_anchor=nv, context=ctx).out for h in range(H)])
    say(f"[fp8] {name}: vs oracle fp8 rel_l2={err:.3e} max_abs={mab:.2e}; "
        f"(the fp8 layer differs from the bf16-logit layer by rel_l2={rel_l2(want, plain):.3e})")
    assert err <= 1e-2 and mab <= 3e-2


def test_fp8_layer_equals_composed_steps():
    q, k, v, b, topk, _ = _case("draft")
    H, N, d = q.shape
    dt = torch.bfloat16
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    g = L.spark_reblock(qd, kd, vd, b)
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, b)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
    steps = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"], fp8=True)
    layer = L.spark_layer(qd, kd, vd, b, topk, fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(steps, layer)
    assert bool(torch.isfinite(layer.float()).all())
