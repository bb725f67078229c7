"""ctypes binding of libspark (include/spark.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of libspark.so.  PyTorch provides device memory (outputs and workspaces are
torch tensors) and the current stream.  There is no fallback: if the library
is missing, or a tensor is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspark.so")

SPARK_F32, SPARK_BF16 = 0, 1
LAYOUT_REBLOCK, LAYOUT_IDENTITY, LAYOUT_GIVEN, LAYOUT_Q_REUSE_K = 0x0, 0x1, 0x2, 0x3
SUMMARY_REWEIGHT, SUMMARY_MEAN = 0x0, 0x4
CONTEXT_EXACT = 0x8
EXACT_FP8 = 0x10
ATTN_ONE_BLOCK = 0x20
OP_REBLOCK, OP_SELECT, OP_SUMMARIZE, OP_ATTN, OP_SPLIT, OP_LAYER = range(6)
_LAYOUTS = {"reblock": LAYOUT_REBLOCK, "identity": LAYOUT_IDENTITY, "given": LAYOUT_GIVEN,
            "q_reuse_k": LAYOUT_Q_REUSE_K}
_SUMMARIES = {"reweight": SUMMARY_REWEIGHT, "mean": SUMMARY_MEAN}

EXPORTED = [
    "spark_version", "spark_status_string", "spark_last_error", "spark_block_count",
    "spark_topk_from_ratio", "spark_workspace_bytes", "spark_reblock", "spark_select",
    "spark_summarize", "spark_attn", "spark_layer", "spark_moments", "spark_msqrt",
    "spark_whiten", "spark_split", "spark_gather", "spark_diagnostics", "spark_quant_e4m3",
    "spark_debug_partition_ws_bytes", "spark_debug_partition_level", "spark_debug_argmin",
    "spark_mfma_peak_probe", "spark_attn_noalloc", "spark_attn_noalloc_scratch_bytes",
]


class SparkArgs(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_anchor", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_int32)]


class SparkError(RuntimeError):
    pass


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t
_A = ctypes.POINTER(SparkArgs)


def lib() -> ctypes.CDLL:
    """Load libspark.so (built by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SparkError(f"{LIB_PATH} is missing: build it with "
                         "`python -m block_sparse_attention_mahalanobis_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "spark_version": ([], ctypes.c_int),
        "spark_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "spark_last_error": ([], ctypes.c_char_p),
        "spark_block_count": ([_I, _I], ctypes.c_int),
        "spark_topk_from_ratio": ([ctypes.c_double, _I], ctypes.c_int),
        "spark_workspace_bytes": ([_A, ctypes.c_int, _I], _Z),
        "spark_reblock": ([_A, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
        "spark_select": ([_A, _P, _P, _P, _I, _P, _P, _P], ctypes.c_int),
        "spark_summarize": ([_A, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
        "spark_attn": ([_A, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
        "spark_layer": ([_A, _P, _P, _P, _I, _P, _P, _Z, _P], ctypes.c_int),
        "spark_moments": ([_A, _P, _P, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
        "spark_msqrt": ([_I, _I, _P, _P, _P, _Z, _P], ctypes.c_int),
        "spark_whiten": ([_A, _I, _P, _P, _P, _P], ctypes.c_int),
        "spark_split": ([_A, _I, _P, _P, _P, _Z, _P], ctypes.c_int),
        "spark_gather": ([_A, _P, _P, _P, _P, _P, _P], ctypes.c_int),
        "spark_diagnostics": ([_A, _P, _P, _P, _I, _P, _P, _P, _P, _P], ctypes.c_int),
        "spark_quant_e4m3": ([_I, _I, _I, _I, _P, _P, _P, _P], ctypes.c_int),
        "spark_debug_partition_ws_bytes": ([_I, _I, _I], _Z),
        "spark_debug_partition_level": ([_I, _I, _I, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
        "spark_debug_argmin": ([_I, _I, _P, _P, _P, _P], ctypes.c_int),
        "spark_mfma_peak_probe": ([_I, _I, _P, _P], ctypes.c_double),
        "spark_attn_noalloc": ([_A, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P], ctypes.c_int),
        "spark_attn_noalloc_scratch_bytes": ([], _Z),
    }
    for name, (argt, rest) in sig.items():
        f = getattr(L, name)
        f.argtypes = argt
        f.restype = rest
    _lib = L
    return L


def last_error() -> str:
    return lib().spark_last_error().decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise SparkError(f"{what}: {lib().spark_status_string(rc).decode()} ({rc}): {last_error()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise SparkError("libspark needs device tensors")
    if not t.is_contiguous():
        raise SparkError("libspark needs contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return SPARK_F32
    if dt == torch.bfloat16:
        return SPARK_BF16
    raise SparkError(f"unsupported dtype {dt}")


def make_args(H: int, N: int, d: int, block: int, dtype, n_anchor: Optional[int] = None,
              layout: str = "reblock", summary: str = "reweight", context: bool = False,
              fp8: bool = False, one_block: bool = False) -> SparkArgs:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return SparkArgs(H, N, d, block, code, N if n_anchor is None else n_anchor,
                     _LAYOUTS[layout] | _SUMMARIES[summary] | (CONTEXT_EXACT if context else 0)
                     | (EXACT_FP8 if fp8 else 0) | (ATTN_ONE_BLOCK if one_block else 0), 0)


def n_blocks(N: int, block: int) -> int:
    return -(-N // block)


def geometry(N: int, block: int, n_anchor: Optional[int] = None, context: bool = False):
    """(video tokens, video blocks, blocks of q_p / k_p / v_pt): with the
    context mode the tokens from n_anchor on form extra blocks after the
    video blocks; otherwise every token is a video token."""
    nv = n_anchor if (context and n_anchor is not None) else N
    nb = n_blocks(nv, block)
    return nv, nb, nb + n_blocks(N - nv, block)


def topk_from_ratio(ratio: float, nb: int) -> int:
    rc = lib().spark_topk_from_ratio(float(ratio), int(nb))
    _check(rc if rc < 0 else 0, "spark_topk_from_ratio")
    return rc


def workspace_bytes(args: SparkArgs, op: int, topk: int = 0) -> int:
    n = lib().spark_workspace_bytes(ctypes.byref(args), op, topk)
    if n == ctypes.c_size_t(-1).value:
        raise SparkError(f"spark_workspace_bytes: {last_error()}")
    return n


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# the four steps
# ---------------------------------------------------------------------------

def spark_reblock(q, k, v, block: int, layout: str = "reblock", perm_q=None, perm_k=None,
                  n_anchor: Optional[int] = None, want_q_p: bool = True, context: bool = False):
    """Reblock + gather + pool.  Returns a dict of device tensors: perm_q,
    perm_k [H,N] int32, q_p, k_p [H,Np,d], v_pt [H,nbt,d,block], qbar, kbar
    [H,nb,d] fp32, anchor [H,d] fp32 (nb video blocks, nbt = nb + context
    blocks, Np = nbt * block)."""
    H, N, d = q.shape
    dev = q.device
    _, nb, nbt = geometry(N, block, n_anchor, context)
    Np = nbt * block
    a = make_args(H, N, d, block, q.dtype, n_anchor, layout, context=context)
    if layout == "given":
        perm_q = perm_q.to(device=dev, dtype=torch.int32).contiguous()
        perm_k = perm_k.to(device=dev, dtype=torch.int32).contiguous()
    else:
        perm_q = torch.empty((H, N), dtype=torch.int32, device=dev)
        perm_k = torch.empty((H, N), dtype=torch.int32, device=dev)
    out = dict(
        perm_q=perm_q, perm_k=perm_k,
        q_p=torch.empty((H, Np, d), dtype=q.dtype, device=dev) if want_q_p else None,
        k_p=torch.empty((H, Np, d), dtype=q.dtype, device=dev),
        v_pt=torch.empty((H, nbt, d, block), dtype=q.dtype, device=dev),
        qbar=torch.empty((H, nb, d), dtype=torch.float32, device=dev),
        kbar=torch.empty((H, nb, d), dtype=torch.float32, device=dev),
        anchor=torch.empty((H, d), dtype=torch.float32, device=dev),
    )
    nws = workspace_bytes(a, OP_REBLOCK)
    ws = _ws(nws, dev)
    _check(lib().spark_reblock(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(perm_q), _ptr(perm_k),
                               _ptr(out["q_p"]), _ptr(out["k_p"]), _ptr(out["v_pt"]), _ptr(out["qbar"]),
                               _ptr(out["kbar"]), _ptr(out["anchor"]), _ptr(ws), nws, _stream()),
           "spark_reblock")
    return out


def spark_select(qbar, kbar, topk: int, N: int, block: int, scores_in=None, want_scores=False,
                 dtype=torch.bfloat16, n_anchor: Optional[int] = None, context: bool = False):
    """idx [H, nb, topk] int32 (ascending) and, if asked, the scores used."""
    ref = qbar if qbar is not None else scores_in
    H = ref.shape[0]
    d = qbar.shape[2] if qbar is not None else 128
    _, nb, _ = geometry(N, block, n_anchor, context)
    a = make_args(H, N, d, block, dtype, n_anchor, context=context)
    idx = torch.empty((H, nb, topk), dtype=torch.int32, device=ref.device)
    sc = torch.empty((H, nb, nb), dtype=torch.float32, device=ref.device) if want_scores else None
    _check(lib().spark_select(ctypes.byref(a), _ptr(qbar), _ptr(kbar), _ptr(scores_in), topk, _ptr(idx),
                              _ptr(sc), _stream()), "spark_select")
    return (idx, sc) if want_scores else idx


def spark_summarize(k_p, v_pt, anchor, N: int, block: int, summary: str = "reweight",
                    n_anchor: Optional[int] = None, context: bool = False):
    """ksum, vsum [H, nb, d] fp32 and bias [H, nb] fp32."""
    H, _, d = k_p.shape
    _, nb, _ = geometry(N, block, n_anchor, context)
    a = make_args(H, N, d, block, k_p.dtype, n_anchor, summary=summary, context=context)
    dev = k_p.device
    ksum = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
    vsum = torch.empty((H, nb, d), dtype=torch.float32, device=dev)
    bias = torch.empty((H, nb), dtype=torch.float32, device=dev)
    _check(lib().spark_summarize(ctypes.byref(a), _ptr(k_p), _ptr(v_pt), _ptr(anchor), _ptr(ksum),
                                 _ptr(vsum), _ptr(bias), _stream()), "spark_summarize")
    return ksum, vsum, bias


def spark_attn(q_p, k_p, v_pt, idx, ksum, vsum, bias, N: int, block: int, perm_q=None, out=None,
               ws=None, n_anchor: Optional[int] = None, context: bool = False, fp8: bool = False,
               one_block: bool = False):
    """Fused two-branch attention; [H, N, d] in original order if perm_q is
    given, else [H, Np, d] in permuted order.  fp8: E4M3 logits.  one_block:
    one query block per workgroup (SPARK_ATTN_ONE_BLOCK)."""
    H, Np, d = q_p.shape
    topk = idx.shape[2]
    a = make_args(H, N, d, block, q_p.dtype, n_anchor, context=context, fp8=fp8, one_block=one_block)
    dev = q_p.device
    if out is None:
        out = torch.empty((H, N if perm_q is not None else Np, d), dtype=q_p.dtype, device=dev)
    nws = workspace_bytes(a, OP_ATTN)
    if ws is None:
        ws = _ws(nws, dev)
    _check(lib().spark_attn(ctypes.byref(a), _ptr(q_p), _ptr(k_p), _ptr(v_pt), _ptr(idx), topk, _ptr(ksum),
                            _ptr(vsum), _ptr(bias), _ptr(perm_q), _ptr(out), _ptr(ws), nws, _stream()),
           "spark_attn")
    return out


def spark_attn_noalloc(q_p, k_p, v_pt, idx, ksum, vsum, bias, N: int, block: int, perm_q=None, out=None,
                       n_anchor: Optional[int] = None, context: bool = False, fp8: bool = False,
                       one_block: bool = False):
    """spark_attn with its scratch in the library's fixed device array (no
    workspace argument, nothing allocated by the library)."""
    H, Np, d = q_p.shape
    topk = idx.shape[2]
    a = make_args(H, N, d, block, q_p.dtype, n_anchor, context=context, fp8=fp8, one_block=one_block)
    if out is None:
        out = torch.empty((H, N if perm_q is not None else Np, d), dtype=q_p.dtype, device=q_p.device)
    _check(lib().spark_attn_noalloc(ctypes.byref(a), _ptr(q_p), _ptr(k_p), _ptr(v_pt), _ptr(idx), topk,
                                    _ptr(ksum), _ptr(vsum), _ptr(bias), _ptr(perm_q), _ptr(out), _stream()),
           "spark_attn_noalloc")
    return out


def spark_diagnostics(q_p, k_p, idx, ksum, bias, N: int, block: int):
    """Per-query attention-mass recall and log-mass error, [H, N] fp32 each,
    in the permuted order of q_p."""
    H, Np, d = q_p.shape
    topk = idx.shape[2]
    a = make_args(H, N, d, block, q_p.dtype)
    recall = torch.empty((H, N), dtype=torch.float32, device=q_p.device)
    logmass = torch.empty((H, N), dtype=torch.float32, device=q_p.device)
    _check(lib().spark_diagnostics(ctypes.byref(a), _ptr(q_p), _ptr(k_p), _ptr(idx), topk, _ptr(ksum),
                                   _ptr(bias), _ptr(recall), _ptr(logmass), _stream()),
           "spark_diagnostics")
    return recall, logmass


def spark_layer(q, k, v, block: int, topk: int, layout: str = "reblock", summary: str = "reweight",
                n_anchor: Optional[int] = None, out=None, ws=None, context: bool = False,
                fp8: bool = False, one_block: bool = False):
    """The whole layer in one call; intermediates live in the workspace."""
    H, N, d = q.shape
    a = make_args(H, N, d, block, q.dtype, n_anchor, layout, summary, context, fp8, one_block)
    nws = workspace_bytes(a, OP_LAYER, topk)
    if ws is None:
        ws = _ws(nws, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(lib().spark_layer(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), topk, _ptr(out), _ptr(ws), nws,
                             _stream()), "spark_layer")
    return out


# ---------------------------------------------------------------------------
# stages
# ---------------------------------------------------------------------------

def spark_moments(q, k, n_anchor: Optional[int] = None):
    H, N, d = q.shape
    a = make_args(H, N, d, 128, q.dtype, n_anchor)
    dev = q.device
    MQ = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    MK = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    anchor = torch.empty((H, d), dtype=torch.float32, device=dev)
    nws = workspace_bytes(a, OP_REBLOCK)
    ws = _ws(nws, dev)
    _check(lib().spark_moments(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(MQ), _ptr(MK), _ptr(anchor), _ptr(ws),
                               nws, _stream()), "spark_moments")
    return MQ, MK, anchor


def spark_msqrt(M):
    count, d, _ = M.shape
    W = torch.empty_like(M)
    _check(lib().spark_msqrt(count, d, _ptr(M), _ptr(W), None, 0, _stream()), "spark_msqrt")
    return W


def spark_whiten(x, W):
    count, N, d = x.shape
    a = make_args(1, N, d, 128, x.dtype)
    xh = torch.empty_like(x)
    _check(lib().spark_whiten(ctypes.byref(a), count, _ptr(x), _ptr(W), _ptr(xh), _stream()), "spark_whiten")
    return xh


def spark_split(xhat, block: int):
    count, N, d = xhat.shape
    a = make_args((count + 1) // 2, N, d, block, xhat.dtype)
    perm = torch.empty((count, N), dtype=torch.int32, device=xhat.device)
    nws = workspace_bytes(a, OP_SPLIT)
    ws = _ws(nws, xhat.device)
    _check(lib().spark_split(ctypes.byref(a), count, _ptr(xhat), _ptr(perm), _ptr(ws), nws, _stream()),
           "spark_split")
    return perm


def spark_gather(x, perm, block: int, want_rows=True, want_transposed=False, want_means=True):
    H, N, d = x.shape
    nb = n_blocks(N, block)
    a = make_args(H, N, d, block, x.dtype)
    dev = x.device
    xp = torch.empty((H, nb * block, d), dtype=x.dtype, device=dev) if want_rows else None
    xpt = torch.empty((H, nb, d, block), dtype=x.dtype, device=dev) if want_transposed else None
    xbar = torch.empty((H, nb, d), dtype=torch.float32, device=dev) if want_means else None
    perm = perm.to(device=dev, dtype=torch.int32).contiguous()
    _check(lib().spark_gather(ctypes.byref(a), _ptr(x), _ptr(perm), _ptr(xp), _ptr(xpt), _ptr(xbar), _stream()),
           "spark_gather")
    return xp, xpt, xbar


def spark_quant_e4m3(x, group: int):
    """E4M3 bytes [rows, d] (uint8) and per-group power-of-two scales of the
    rows of x [rows, d] (bf16 or fp32), groups of ``group`` rows."""
    rows, d = x.shape
    x8 = torch.empty((rows, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((-(-rows // group),), dtype=torch.float32, device=x.device)
    _check(lib().spark_quant_e4m3(rows, d, group, _dtype_code(x.dtype), _ptr(x), _ptr(x8), _ptr(scales),
                                  _stream()), "spark_quant_e4m3")
    return x8, scales


def spark_debug_partition_level(s, ids, block: int):
    """One capacity partition per row of s [count, n] fp32 with ids [count, n]
    int32 (ascending per row): left child's ids then the right child's."""
    count, n = s.shape
    nws = lib().spark_debug_partition_ws_bytes(count, n, block)
    if nws == ctypes.c_size_t(-1).value:
        raise SparkError(f"spark_debug_partition_ws_bytes: {last_error()}")
    ws = _ws(nws, s.device)
    out = torch.empty((count, n), dtype=torch.int32, device=s.device)
    _check(lib().spark_debug_partition_level(count, n, block, _ptr(s), _ptr(ids), _ptr(out), _ptr(ws), nws,
                                             _stream()), "spark_debug_partition_level")
    return out


def spark_debug_argmin(vals, ids):
    """Per row of vals [count, n] fp32 / ids [count, n] int32: the id of the
    minimum (-0 = +0, NaN last, ties to the lower id)."""
    count, n = vals.shape
    out = torch.empty((count,), dtype=torch.int32, device=vals.device)
    _check(lib().spark_debug_argmin(count, n, _ptr(vals), _ptr(ids), _ptr(out), _stream()), "spark_debug_argmin")
    return out


def mfma_peak_tflops(workgroups: int = 512, iters: int = 16384, repeats: int = 5) -> float:
    """Sustained bf16 MFMA rate of this GPU (TFLOP/s): the best of `repeats`
    event-timed launches of the library's register-only MFMA loop."""
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda:0")
    best = 0.0
    for _ in range(repeats + 1):                      # the first launch warms up
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = lib().spark_mfma_peak_probe(workgroups, iters, _ptr(sink), _stream())
        e1.record()
        if flops < 0:
            raise SparkError(f"spark_mfma_peak_probe: {last_error()}")
        torch.cuda.synchronize()
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best
