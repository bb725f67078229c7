"""spark_attn_noalloc -- spark_attn with its scratch in the library's fixed
per-GPU device array instead of a caller workspace (for callers that cannot
allocate) -- against spark_attn on the same inputs, bit for bit (the same
kernels run on the same operands), on consecutive calls whose second input
is smaller than the first (the array keeps the earlier call's contents),
over the three attention kernels (d = 128 block 128, the block-64 MFMA
kernel, the fp32 generic kernel), plus E4M3 logits at a size that fits.
Arguments that need more scratch than the array holds are rejected before
anything is enqueued (checked without a GPU)."""
import ctypes

import numpy as np
import pytest
import torch

from block_sparse_attention_mahalanobis_amd import _lib as L
from block_sparse_attention_mahalanobis_amd.workload import WORKLOADS, make_workload

DEV = "cuda:0"
FAKE = ctypes.c_void_p(0x10000)


def _inputs(name):
    if name == "draft_b128":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[0, 1, 2])
        return q, k, v, torch.bfloat16, 128, 0.1
    if name == "draft_b64_smaller":
        q, k, v = make_workload(WORKLOADS["draft"], heads=[5])
        return q[:, :9000], k[:, :9000], v[:, :9000], torch.bfloat16, 64, 0.2
    if name == "tiny_f32":
        q, k, v = make_workload(WORKLOADS["tiny"])
        return q[:, :1000], k[:, :1000], v[:, :1000], torch.float32, 64, 0.25
    raise KeyError(name)


def _routed(name):
    q, k, v, dt, b, ratio = _inputs(name)
    H, N, d = q.shape
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dt)
    g = L.spark_reblock(t(q), t(k), t(v), b)
    topk = L.topk_from_ratio(ratio, L.n_blocks(N, b))
    idx = L.spark_select(g["qbar"], g["kbar"], topk, N, b)
    ks, vs, bias = L.spark_summarize(g["k_p"], g["v_pt"], g["anchor"], N, b)
    return g, idx, ks, vs, bias, N, b


@pytest.mark.gpu
def test_noalloc_equals_spark_attn_on_consecutive_calls():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    for name in ("draft_b128", "draft_b64_smaller", "tiny_f32"):
        print(f"[noalloc] {name}", flush=True)
        g, idx, ks, vs, bias, N, b = _routed(name)
        want = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
        got = L.spark_attn_noalloc(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"])
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got.float()).all())
        assert torch.equal(got, want), name
        # permuted-order output (no scatter) as well
        want_p = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b)
        got_p = L.spark_attn_noalloc(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b)
        torch.cuda.synchronize()
        assert torch.equal(got_p, want_p), name


@pytest.mark.gpu
def test_noalloc_fp8_logits_equal_spark_attn():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L.lib()
    g, idx, ks, vs, bias, N, b = _routed("draft_b128")
    want = L.spark_attn(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"], fp8=True)
    got = L.spark_attn_noalloc(g["q_p"], g["k_p"], g["v_pt"], idx, ks, vs, bias, N, b, perm_q=g["perm_q"],
                               fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_noalloc_rejects_what_does_not_fit():
    """No GPU needed: validation and the size check run before any device
    call.  The 768p layer fits; its E4M3-logit form (1.3 GB of quantised
    keys) does not."""
    lib = L.lib()
    cap = lib.spark_attn_noalloc_scratch_bytes()
    assert cap == 64 << 20
    H, N, d, b = 40, 245952, 128, 128
    nb = L.n_blocks(N, b)
    plain = L.make_args(H, N, d, b, torch.bfloat16)
    assert L.workspace_bytes(plain, L.OP_ATTN) <= cap
    big = L.make_args(H, N, d, b, torch.bfloat16, fp8=True)
    assert L.workspace_bytes(big, L.OP_ATTN) > cap
    rc = lib.spark_attn_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 193, FAKE, FAKE, FAKE, None, FAKE,
                                None)
    assert rc == -5 and "allocation-free" in L.last_error()
    assert lib.spark_attn_noalloc(ctypes.byref(plain), FAKE, FAKE, FAKE, FAKE, nb + 1, FAKE, FAKE, FAKE, None,
                                  FAKE, None) == -2
    assert lib.spark_attn_noalloc(ctypes.byref(plain), FAKE, None, FAKE, FAKE, 193, FAKE, FAKE, FAKE, None,
                                  FAKE, None) == -1
