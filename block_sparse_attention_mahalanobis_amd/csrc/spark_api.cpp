// libspark host side: argument validation, workspace planning and the launch
// sequence of each entry point of include/spark.h.  Everything is enqueued on
// the caller's stream; nothing is allocated or synchronised here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.hpp"

namespace spark {
// kernels (k_*.hip)
int attn_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* qp, const void* kp,
                const void* vpt, const int32_t* idx, int topk, const float* ksum,
                const float* vsum, const float* bias, const int32_t* perm_q, void* out, void* ws,
                bool fp8, bool paired, hipStream_t st);
size_t attn_ws_bytes(int H, int N, int Nv, int D, int BK, int dtype, bool fp8);
bool attn_fp8_supported(int H, int N, int Nv, int D, int BK, int dtype);
int quant_e4m3_launch(int H, long in_rows, long out_rows, int D, int G, int dtype, const void* x,
                      uint8_t* x8, float* scales, hipStream_t st);
bool attn_uses_mfma(int dtype, int BK);
int gather_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* x,
                  const int32_t* perm, void* xp, void* xpt, float* xbar, hipStream_t st);
int summarize_launch(int H, int N, int nbc, int D, int BK, int dtype, const void* kp,
                     const void* vpt, const float* anchor, float* ksum, float* vsum, float* bias,
                     int mean_mode, hipStream_t st);
int anchor_launch(int H, int N, int D, int dtype, const void* q, float* anchor, int n_anchor,
                  float* scratch, int scratch_nb, hipStream_t st);
int select_launch(int H, int N, int D, int BK, const float* qbar, const float* kbar,
                  const float* scores_in, int topk, int32_t* idx, float* scores_out,
                  hipStream_t st);
size_t moments_ws_bytes(int H, int N, int D);
int moments_launch(int H, int N, int D, int dtype, const void* q, const void* k, float* MQ,
                   float* MK, float* anchor, int n_anchor, void* ws, hipStream_t st);
int copy_perm_launch(long count, const int32_t* src, int32_t* dst, hipStream_t st);
int msqrt_launch(int count, int D, const float* M, float* W, hipStream_t st);
int whiten_launch(int count, int N, int xrows, int D, int dtype, const void* x, const float* W,
                  void* xh, hipStream_t st, float* cpart, int tree_off);
size_t split_ws_bytes(int count, int N, int D, int BK, int dtype);
int split_launch(int count, int N, int D, int BK, int dtype, const void* xh, int32_t* perm_lo,
                 int32_t* perm_hi, int split_at, long perm_ld, void* ws, hipStream_t st,
                 bool level0_given);
float* split_level0_partials(void* ws, int count, int N, int D, int BK, int dtype);
int iota_launch(int count, int n, long ld, int from, int32_t* lo, int32_t* hi, int split_at,
                hipStream_t st);
int debug_argmin_launch(int count, int n, const float* vals, const int32_t* ids, int32_t* out,
                        hipStream_t st);
size_t debug_partition_ws_bytes(int count, int n, int BK);
int debug_partition_launch(int count, int n, int BK, const float* s, const int32_t* ids_in,
                           int32_t* ids_out, void* ws, hipStream_t st);
int mfma_peak_launch(int workgroups, int iters, float* sink, hipStream_t st);
size_t noalloc_scratch_bytes();
int attn_noalloc_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* qp, const void* kp,
                        const void* vpt, const int32_t* idx, int topk, const float* ksum,
                        const float* vsum, const float* bias, const int32_t* perm_q, void* out,
                        bool fp8, bool paired, hipStream_t st);
int diag_launch(int H, int N, int D, int BK, int dtype, const void* qp, const void* kp,
                const int32_t* idx, int topk, const float* ksum, const float* bias, float* recall,
                float* logmass, hipStream_t st);
}  // namespace spark

using namespace spark;

// ---- errors -------------------------------------------------------------------
static thread_local char g_err[512] = "";

int spark_set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int spark_check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return spark_set_error(SPARK_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return SPARK_OK;
}

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int esize(int dtype) { return dtype == SPARK_BF16 ? 2 : 4; }

int check_ptr(const void* p, const char* fn, const char* name, bool nullable = false) {
  if (p == nullptr) {
    if (nullable) return SPARK_OK;
    return spark_set_error(SPARK_E_ARG, "%s: %s is NULL", fn, name);
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return spark_set_error(SPARK_E_ARG, "%s: %s is not 16-byte aligned", fn, name);
  return SPARK_OK;
}

#define CHECK(x)            \
  do {                      \
    const int _rc = (x);    \
    if (_rc) return _rc;    \
  } while (0)

int check_args(const spark_args* a, const char* fn) {
  if (a == nullptr) return spark_set_error(SPARK_E_ARG, "%s: args is NULL", fn);
  if (a->reserved != 0) return spark_set_error(SPARK_E_ARG, "%s: args.reserved must be 0", fn);
  if (a->dtype != SPARK_F32 && a->dtype != SPARK_BF16)
    return spark_set_error(SPARK_E_DTYPE, "%s: dtype %d is not SPARK_F32/SPARK_BF16", fn, a->dtype);
  if (a->d != 64 && a->d != 128)
    return spark_set_error(SPARK_E_UNSUPPORTED, "%s: head dim %d not in {64, 128}", fn, a->d);
  if (a->H < 1) return spark_set_error(SPARK_E_SHAPE, "%s: H=%d < 1", fn, a->H);
  if (a->N < 1) return spark_set_error(SPARK_E_SHAPE, "%s: N=%d < 1", fn, a->N);
  if (a->block < 1 || a->block > 128)
    return spark_set_error(SPARK_E_SHAPE, "%s: block=%d not in [1, 128]", fn, a->block);
  if (a->n_anchor < 1 || a->n_anchor > a->N)
    return spark_set_error(SPARK_E_SHAPE, "%s: n_anchor=%d not in [1, N=%d]", fn, a->n_anchor, a->N);
  const uint32_t layout = a->flags & SPARK_LAYOUT_MASK;
  if (layout > SPARK_LAYOUT_Q_REUSE_K ||
      (a->flags & ~(SPARK_LAYOUT_MASK | SPARK_SUMMARY_MEAN | SPARK_CONTEXT_EXACT | SPARK_EXACT_FP8 |
                    SPARK_ATTN_ONE_BLOCK)))
    return spark_set_error(SPARK_E_ARG, "%s: bad flags 0x%x", fn, a->flags);
  const long nb = (a->N + (long)a->block - 1) / a->block;
  if ((long)a->H * nb > 0x7fffffffL || (long)a->N * a->d > 0x7fffffffL)
    return spark_set_error(SPARK_E_SHAPE, "%s: problem too large", fn);
  return SPARK_OK;
}

// Token geometry: Nv video tokens in nb blocks (all N tokens unless
// SPARK_CONTEXT_EXACT), then nbc context blocks; nbt = nb + nbc blocks in
// q_p / k_p / v_pt.
struct Geo {
  int Nv, nb, nbc, nbt;
};
Geo geo(const spark_args* a) {
  Geo g;
  g.Nv = (a->flags & SPARK_CONTEXT_EXACT) ? a->n_anchor : a->N;
  g.nb = (g.Nv + a->block - 1) / a->block;
  g.nbc = (a->N - g.Nv + a->block - 1) / a->block;
  g.nbt = g.nb + g.nbc;
  return g;
}

int nblocks(const spark_args* a) { return geo(a).nb; }

bool fp8_of(const spark_args* a) { return (a->flags & SPARK_EXACT_FP8) != 0; }

// SPARK_EXACT_FP8 runs on the d = 128, block 128 bf16 kernel only
int check_fp8(const spark_args* a, const char* fn) {
  if (!fp8_of(a)) return SPARK_OK;
  const Geo g = geo(a);
  if (!attn_fp8_supported(a->H, a->N, g.Nv, a->d, a->block, a->dtype))
    return spark_set_error(SPARK_E_UNSUPPORTED,
                           "%s: SPARK_EXACT_FP8 needs bf16, d = 128, block = 128 and at most 4096 video blocks", fn);
  return SPARK_OK;
}

int reject_context(const spark_args* a, const char* fn) {
  if (a->flags & SPARK_CONTEXT_EXACT)
    return spark_set_error(SPARK_E_UNSUPPORTED, "%s: SPARK_CONTEXT_EXACT is not supported here", fn);
  return SPARK_OK;
}

// The whitening pass can hand the split its root partial centroid sums when
// a 128-row whitening round is exactly one block (bf16, d = 128, block 128).
static bool level0_fusable(const spark_args* a) {
  return a->dtype == SPARK_BF16 && a->d == 128 && a->block == 128;
}

size_t reblock_ws(const spark_args* a) {
  const uint32_t layout = a->flags & SPARK_LAYOUT_MASK;
  if (layout != SPARK_LAYOUT_REBLOCK && layout != SPARK_LAYOUT_Q_REUSE_K) return 0;
  const int H = a->H, N = a->N, D = a->d, Nv = geo(a).Nv;
  size_t b = 0;
  b += up((size_t)2 * H * D * D * 4);                     // moments [MK | MQ]
  b += up((size_t)2 * H * D * D * 4);                     // roots  [W_Q | W_K]
  b += up(moments_ws_bytes(H, N, D));
  b += up((size_t)2 * H * Nv * D * esize(a->dtype));      // whitened (video) rows
  b += up(split_ws_bytes(2 * H, Nv, D, a->block, a->dtype));
  return b;
}

struct LayerBufs {
  int32_t *perm_q, *perm_k, *idx;
  void *q_p, *k_p, *v_pt;
  float *qbar, *kbar, *anchor, *ksum, *vsum, *bias;
  void* scratch;
};

size_t layer_bufs(const spark_args* a, int topk, char* base, LayerBufs* o) {
  const Geo g = geo(a);
  const int H = a->H, N = a->N, D = a->d, nb = g.nb;
  const size_t Np = (size_t)g.nbt * a->block;
  const int es = esize(a->dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += up(bytes);
    return p;
  };
  LayerBufs b;
  b.perm_q = (int32_t*)take((size_t)H * N * 4);
  b.perm_k = (int32_t*)take((size_t)H * N * 4);
  b.q_p = take((size_t)H * Np * D * es);
  b.k_p = take((size_t)H * Np * D * es);
  b.v_pt = take((size_t)H * Np * D * es);   // [H, nbt, D, block]
  b.qbar = (float*)take((size_t)H * nb * D * 4);
  b.kbar = (float*)take((size_t)H * nb * D * 4);
  b.anchor = (float*)take((size_t)H * D * 4);
  b.idx = (int32_t*)take((size_t)H * nb * (size_t)topk * 4);
  b.ksum = (float*)take((size_t)H * nb * D * 4);
  b.vsum = (float*)take((size_t)H * nb * D * 4);
  b.bias = (float*)take((size_t)H * nb * 4);
  b.scratch = take(0);
  if (o) *o = b;
  return off + std::max(reblock_ws(a), attn_ws_bytes(H, N, g.Nv, D, a->block, a->dtype, fp8_of(a)));
}

}  // namespace

// ---- utilities -----------------------------------------------------------------
extern "C" {

int spark_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* spark_status_string(int s) {
  switch (s) {
    case SPARK_OK: return "SPARK_OK";
    case SPARK_E_ARG: return "SPARK_E_ARG";
    case SPARK_E_SHAPE: return "SPARK_E_SHAPE";
    case SPARK_E_DTYPE: return "SPARK_E_DTYPE";
    case SPARK_E_UNSUPPORTED: return "SPARK_E_UNSUPPORTED";
    case SPARK_E_WORKSPACE: return "SPARK_E_WORKSPACE";
    case SPARK_E_HIP: return "SPARK_E_HIP";
    default: return "SPARK_E_UNKNOWN";
  }
}

const char* spark_last_error(void) { return g_err; }

int spark_block_count(int32_t N, int32_t block) {
  if (N < 1 || block < 1) return spark_set_error(SPARK_E_SHAPE, "spark_block_count: N=%d block=%d", N, block);
  return (int)(((long)N + block - 1) / block);
}

int spark_topk_from_ratio(double ratio, int32_t n_blocks) {
  if (n_blocks < 1) return spark_set_error(SPARK_E_SHAPE, "spark_topk_from_ratio: n_blocks=%d", n_blocks);
  if (!std::isfinite(ratio)) return spark_set_error(SPARK_E_ARG, "spark_topk_from_ratio: ratio not finite");
  const double k = std::ceil(ratio * (double)n_blocks - 1e-9);
  if (k < 1.0) return 1;
  if (k > (double)n_blocks) return n_blocks;
  return (int)k;
}

size_t spark_workspace_bytes(const spark_args* a, int op, int32_t topk) {
  if (check_args(a, "spark_workspace_bytes")) return (size_t)-1;
  const int nb = nblocks(a);
  switch (op) {
    case SPARK_OP_REBLOCK: return reblock_ws(a);
    case SPARK_OP_SELECT: return 0;
    case SPARK_OP_SUMMARIZE: return 0;
    case SPARK_OP_ATTN: return attn_ws_bytes(a->H, a->N, geo(a).Nv, a->d, a->block, a->dtype, fp8_of(a));
    case SPARK_OP_SPLIT: return split_ws_bytes(2 * a->H, a->N, a->d, a->block, a->dtype);
    case SPARK_OP_LAYER:
      if (topk < 1 || topk > nb) {
        spark_set_error(SPARK_E_SHAPE, "spark_workspace_bytes: topk=%d not in [1, %d]", topk, nb);
        return (size_t)-1;
      }
      return layer_bufs(a, topk, nullptr, nullptr);
    default:
      spark_set_error(SPARK_E_ARG, "spark_workspace_bytes: unknown op %d", op);
      return (size_t)-1;
  }
}

// ---- stages ------------------------------------------------------------------------
int spark_moments(const spark_args* a, const void* q, const void* k, float* MQ, float* MK,
                  float* anchor, void* ws, size_t ws_bytes, spark_stream_t stream) {
  const char* fn = "spark_moments";
  CHECK(check_args(a, fn));
  CHECK(reject_context(a, fn));
  CHECK(check_ptr(q, fn, "q"));
  CHECK(check_ptr(k, fn, "k"));
  CHECK(check_ptr(MQ, fn, "MQ"));
  CHECK(check_ptr(MK, fn, "MK"));
  CHECK(check_ptr(anchor, fn, "anchor", true));
  CHECK(check_ptr(ws, fn, "ws"));
  if (ws_bytes < moments_ws_bytes(a->H, a->N, a->d))
    return spark_set_error(SPARK_E_WORKSPACE, "%s: ws_bytes %zu < %zu", fn, ws_bytes, moments_ws_bytes(a->H, a->N, a->d));
  return moments_launch(a->H, a->N, a->d, a->dtype, q, k, MQ, MK, anchor, a->n_anchor, ws, (hipStream_t)stream);
}

int spark_msqrt(int32_t count, int32_t d, const float* M, float* W, void* ws, size_t ws_bytes,
                spark_stream_t stream) {
  const char* fn = "spark_msqrt";
  if (count < 1) return spark_set_error(SPARK_E_SHAPE, "%s: count=%d", fn, count);
  if (d != 64 && d != 128) return spark_set_error(SPARK_E_UNSUPPORTED, "%s: d=%d", fn, d);
  CHECK(check_ptr(M, fn, "M"));
  CHECK(check_ptr(W, fn, "W"));
  (void)ws;         // the iteration runs in LDS: no workspace
  (void)ws_bytes;
  return msqrt_launch(count, d, M, W, (hipStream_t)stream);
}

int spark_whiten(const spark_args* a, int32_t count, const void* x, const float* W, void* xhat,
                 spark_stream_t stream) {
  const char* fn = "spark_whiten";
  CHECK(check_args(a, fn));
  CHECK(reject_context(a, fn));
  if (count < 1) return spark_set_error(SPARK_E_SHAPE, "%s: count=%d", fn, count);
  CHECK(check_ptr(x, fn, "x"));
  CHECK(check_ptr(W, fn, "W"));
  CHECK(check_ptr(xhat, fn, "xhat"));
  return whiten_launch(count, a->N, a->N, a->d, a->dtype, x, W, xhat, (hipStream_t)stream, nullptr, 0);
}

int spark_split(const spark_args* a, int32_t count, const void* xhat, int32_t* perm, void* ws,
                size_t ws_bytes, spark_stream_t stream) {
  const char* fn = "spark_split";
  CHECK(check_args(a, fn));
  CHECK(reject_context(a, fn));
  if (count < 1) return spark_set_error(SPARK_E_SHAPE, "%s: count=%d", fn, count);
  CHECK(check_ptr(xhat, fn, "xhat"));
  CHECK(check_ptr(perm, fn, "perm"));
  const size_t need = split_ws_bytes(count, a->N, a->d, a->block, a->dtype);
  CHECK(check_ptr(ws, fn, "ws"));
  if (ws_bytes < need) return spark_set_error(SPARK_E_WORKSPACE, "%s: ws_bytes %zu < %zu", fn, ws_bytes, need);
  return split_launch(count, a->N, a->d, a->block, a->dtype, xhat, perm, perm, count, a->N, ws,
                      (hipStream_t)stream, false);
}

int spark_gather(const spark_args* a, const void* x, const int32_t* perm, void* x_p, void* x_pt,
                 float* xbar, spark_stream_t stream) {
  const char* fn = "spark_gather";
  CHECK(check_args(a, fn));
  CHECK(reject_context(a, fn));
  CHECK(check_ptr(x, fn, "x"));
  CHECK(check_ptr(perm, fn, "perm"));
  CHECK(check_ptr(x_p, fn, "x_p", true));
  CHECK(check_ptr(x_pt, fn, "x_pt", true));
  CHECK(check_ptr(xbar, fn, "xbar", true));
  if (!x_p && !x_pt && !xbar) return SPARK_OK;
  return gather_launch(a->H, a->N, a->N, a->d, a->block, a->dtype, x, perm, x_p, x_pt, xbar,
                       (hipStream_t)stream);
}

// ---- the four steps -----------------------------------------------------------------
int spark_reblock(const spark_args* a, const void* q, const void* k, const void* v,
                  int32_t* perm_q, int32_t* perm_k, void* q_p, void* k_p, void* v_pt,
                  float* qbar, float* kbar, float* anchor, void* ws, size_t ws_bytes,
                  spark_stream_t stream) {
  const char* fn = "spark_reblock";
  CHECK(check_args(a, fn));
  CHECK(check_ptr(q, fn, "q"));
  CHECK(check_ptr(k, fn, "k"));
  CHECK(check_ptr(v, fn, "v"));
  CHECK(check_ptr(perm_q, fn, "perm_q"));
  CHECK(check_ptr(perm_k, fn, "perm_k"));
  CHECK(check_ptr(q_p, fn, "q_p", true));
  CHECK(check_ptr(k_p, fn, "k_p"));
  CHECK(check_ptr(v_pt, fn, "v_pt"));
  CHECK(check_ptr(qbar, fn, "qbar"));
  CHECK(check_ptr(kbar, fn, "kbar"));
  CHECK(check_ptr(anchor, fn, "anchor", true));
  const uint32_t layout = a->flags & SPARK_LAYOUT_MASK;
  const size_t need = reblock_ws(a);
  if (need > 0) {
    CHECK(check_ptr(ws, fn, "ws"));
    if (ws_bytes < need) return spark_set_error(SPARK_E_WORKSPACE, "%s: ws_bytes %zu < %zu", fn, ws_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  const int H = a->H, N = a->N, D = a->d, BK = a->block;
  const Geo g = geo(a);
  const int Nv = g.Nv;   // tokens that are partitioned (the video tokens)
  const int32_t *pq = perm_q, *pk = perm_k;
  if (layout == SPARK_LAYOUT_REBLOCK) {
    char* w = (char*)ws;
    float* Ms = (float*)w;  w += up((size_t)2 * H * D * D * 4);   // [MK | MQ]
    float* Ws = (float*)w;  w += up((size_t)2 * H * D * D * 4);   // [W_Q | W_K]
    void* scr = w;          w += up(moments_ws_bytes(H, N, D));
    void* xh = w;           w += up((size_t)2 * H * Nv * D * esize(a->dtype));
    void* sws = w;
    float* MK = Ms;
    float* MQ = Ms + (size_t)H * D * D;
    // moments over all N tokens; queries are whitened by M_K^{1/2} (first H
    // roots), keys by M_Q^{1/2}; only the Nv video rows are whitened and split
    CHECK(moments_launch(H, N, D, a->dtype, q, k, MQ, MK, anchor, a->n_anchor, scr, st));
    CHECK(msqrt_launch(2 * H, D, Ms, Ws, st));
    // bf16, d = 128, block 128: the whitening pass also stores the split's
    // root partial centroid sums (the split then skips that pass)
    float* cp0 = level0_fusable(a) ? split_level0_partials(sws, 2 * H, Nv, D, BK, a->dtype) : nullptr;
    CHECK(whiten_launch(H, Nv, N, D, a->dtype, q, Ws, xh, st, cp0, 0));
    CHECK(whiten_launch(H, Nv, N, D, a->dtype, k, Ws + (size_t)H * D * D,
                        (char*)xh + (size_t)H * Nv * D * esize(a->dtype), st, cp0, H));
    CHECK(split_launch(2 * H, Nv, D, BK, a->dtype, xh, perm_q, perm_k, H, N, sws, st, cp0 != nullptr));
    CHECK(iota_launch(2 * H, N - Nv, N, Nv, perm_q, perm_k, H, st));   // context stays in place
  } else if (layout == SPARK_LAYOUT_Q_REUSE_K) {
    // the same key side as REBLOCK (keys whitened by M_Q^{1/2}); the query
    // moments are still needed for M_Q and the anchor, the key moments not
    char* w = (char*)ws;
    float* Ms = (float*)w;  w += up((size_t)2 * H * D * D * 4);
    float* Ws = (float*)w;  w += up((size_t)2 * H * D * D * 4);
    void* scr = w;          w += up(moments_ws_bytes(H, N, D));
    void* xh = w;           w += up((size_t)2 * H * Nv * D * esize(a->dtype));
    void* sws = w;
    float* MQ = Ms;
    CHECK(moments_launch(H, N, D, a->dtype, q, nullptr, MQ, nullptr, anchor, a->n_anchor, scr, st));
    CHECK(msqrt_launch(H, D, MQ, Ws, st));
    float* cp0 = level0_fusable(a) ? split_level0_partials(sws, H, Nv, D, BK, a->dtype) : nullptr;
    CHECK(whiten_launch(H, Nv, N, D, a->dtype, k, Ws, xh, st, cp0, 0));
    CHECK(split_launch(H, Nv, D, BK, a->dtype, xh, perm_k, perm_k, H, N, sws, st, cp0 != nullptr));
    CHECK(iota_launch(H, N - Nv, N, Nv, perm_k, perm_k, H, st));
    CHECK(copy_perm_launch((long)H * N, perm_k, perm_q, st));
    pq = perm_k;
  } else {
    if (layout == SPARK_LAYOUT_IDENTITY) {
      pq = nullptr;  // gather treats NULL as the identity
      pk = nullptr;
    }
    // qbar (written by the gather below) holds the anchor's chunk sums
    if (anchor) CHECK(anchor_launch(H, N, D, a->dtype, q, anchor, a->n_anchor, qbar, g.nb, st));
  }
  CHECK(gather_launch(H, N, Nv, D, BK, a->dtype, q, pq, q_p, nullptr, qbar, st));
  CHECK(gather_launch(H, N, Nv, D, BK, a->dtype, k, pk, k_p, nullptr, kbar, st));
  CHECK(gather_launch(H, N, Nv, D, BK, a->dtype, v, pk, nullptr, v_pt, nullptr, st));
  if (layout == SPARK_LAYOUT_IDENTITY) CHECK(iota_launch(2 * H, N, N, 0, perm_q, perm_k, H, st));
  return SPARK_OK;
}

int spark_select(const spark_args* a, const float* qbar, const float* kbar, const float* scores_in,
                 int32_t topk, int32_t* idx, float* scores_out, spark_stream_t stream) {
  const char* fn = "spark_select";
  CHECK(check_args(a, fn));
  const int nb = nblocks(a);
  if (topk < 1 || topk > nb) return spark_set_error(SPARK_E_SHAPE, "%s: topk=%d not in [1, %d]", fn, topk, nb);
  CHECK(check_ptr(scores_in, fn, "scores_in", true));
  if (!scores_in) {
    CHECK(check_ptr(qbar, fn, "qbar"));
    CHECK(check_ptr(kbar, fn, "kbar"));
  }
  CHECK(check_ptr(idx, fn, "idx"));
  CHECK(check_ptr(scores_out, fn, "scores_out", true));
  return select_launch(a->H, geo(a).Nv, a->d, a->block, qbar, kbar, scores_in, topk, idx, scores_out,
                       (hipStream_t)stream);
}

int spark_summarize(const spark_args* a, const void* k_p, const void* v_pt, const float* anchor,
                    float* ksum, float* vsum, float* bias, spark_stream_t stream) {
  const char* fn = "spark_summarize";
  CHECK(check_args(a, fn));
  const int mean_mode = (a->flags & SPARK_SUMMARY_MEAN) ? 1 : 0;
  CHECK(check_ptr(k_p, fn, "k_p"));
  CHECK(check_ptr(v_pt, fn, "v_pt"));
  CHECK(check_ptr(anchor, fn, "anchor", mean_mode != 0));
  CHECK(check_ptr(ksum, fn, "ksum"));
  CHECK(check_ptr(vsum, fn, "vsum"));
  CHECK(check_ptr(bias, fn, "bias"));
  const Geo g = geo(a);
  return summarize_launch(a->H, g.Nv, g.nbc, a->d, a->block, a->dtype, k_p, v_pt, anchor, ksum, vsum,
                          bias, mean_mode, (hipStream_t)stream);
}

int spark_attn(const spark_args* a, const void* q_p, const void* k_p, const void* v_pt,
               const int32_t* idx, int32_t topk, const float* ksum, const float* vsum,
               const float* bias, const int32_t* perm_q, void* out, void* ws, size_t ws_bytes,
               spark_stream_t stream) {
  const char* fn = "spark_attn";
  CHECK(check_args(a, fn));
  const int nb = nblocks(a);
  if (topk < 1 || topk > nb) return spark_set_error(SPARK_E_SHAPE, "%s: topk=%d not in [1, %d]", fn, topk, nb);
  CHECK(check_ptr(q_p, fn, "q_p"));
  CHECK(check_ptr(k_p, fn, "k_p"));
  CHECK(check_ptr(v_pt, fn, "v_pt"));
  CHECK(check_ptr(idx, fn, "idx"));
  CHECK(check_ptr(ksum, fn, "ksum"));
  CHECK(check_ptr(vsum, fn, "vsum"));
  CHECK(check_ptr(bias, fn, "bias"));
  CHECK(check_ptr(perm_q, fn, "perm_q", true));
  CHECK(check_ptr(out, fn, "out"));
  CHECK(check_fp8(a, fn));
  const int Nv = geo(a).Nv;
  const size_t need = attn_ws_bytes(a->H, a->N, Nv, a->d, a->block, a->dtype, fp8_of(a));
  if (need > 0) {
    CHECK(check_ptr(ws, fn, "ws"));
    if (ws_bytes < need) return spark_set_error(SPARK_E_WORKSPACE, "%s: ws_bytes %zu < %zu", fn, ws_bytes, need);
  }
  return attn_launch(a->H, a->N, Nv, a->d, a->block, a->dtype, q_p, k_p, v_pt, idx, topk, ksum, vsum,
                     bias, perm_q, out, ws, fp8_of(a), !(a->flags & SPARK_ATTN_ONE_BLOCK), (hipStream_t)stream);
}

size_t spark_attn_noalloc_scratch_bytes(void) { return noalloc_scratch_bytes(); }

int spark_attn_noalloc(const spark_args* a, const void* q_p, const void* k_p, const void* v_pt,
                       const int32_t* idx, int32_t topk, const float* ksum, const float* vsum,
                       const float* bias, const int32_t* perm_q, void* out, spark_stream_t stream) {
  const char* fn = "spark_attn_noalloc";
  CHECK(check_args(a, fn));
  const int nb = nblocks(a);
  if (topk < 1 || topk > nb) return spark_set_error(SPARK_E_SHAPE, "%s: topk=%d not in [1, %d]", fn, topk, nb);
  CHECK(check_ptr(q_p, fn, "q_p"));
  CHECK(check_ptr(k_p, fn, "k_p"));
  CHECK(check_ptr(v_pt, fn, "v_pt"));
  CHECK(check_ptr(idx, fn, "idx"));
  CHECK(check_ptr(ksum, fn, "ksum"));
  CHECK(check_ptr(vsum, fn, "vsum"));
  CHECK(check_ptr(bias, fn, "bias"));
  CHECK(check_ptr(perm_q, fn, "perm_q", true));
  CHECK(check_ptr(out, fn, "out"));
  CHECK(check_fp8(a, fn));
  const int Nv = geo(a).Nv;
  const size_t need = attn_ws_bytes(a->H, a->N, Nv, a->d, a->block, a->dtype, fp8_of(a));
  if (need > noalloc_scratch_bytes())
    return spark_set_error(SPARK_E_WORKSPACE, "%s: these arguments need %zu bytes of scratch; the "
                           "allocation-free entry point holds %zu (use spark_attn with a workspace)",
                           fn, need, noalloc_scratch_bytes());
  return attn_noalloc_launch(a->H, a->N, Nv, a->d, a->block, a->dtype, q_p, k_p, v_pt, idx, topk, ksum, vsum,
                             bias, perm_q, out, fp8_of(a), !(a->flags & SPARK_ATTN_ONE_BLOCK),
                             (hipStream_t)stream);
}

int spark_layer(const spark_args* a, const void* q, const void* k, const void* v, int32_t topk,
                void* out, void* ws, size_t ws_bytes, spark_stream_t stream) {
  const char* fn = "spark_layer";
  CHECK(check_args(a, fn));
  if ((a->flags & SPARK_LAYOUT_MASK) == SPARK_LAYOUT_GIVEN)
    return spark_set_error(SPARK_E_ARG, "%s: SPARK_LAYOUT_GIVEN needs spark_reblock", fn);
  const int nb = nblocks(a);
  if (topk < 1 || topk > nb) return spark_set_error(SPARK_E_SHAPE, "%s: topk=%d not in [1, %d]", fn, topk, nb);
  CHECK(check_fp8(a, fn));
  CHECK(check_ptr(q, fn, "q"));
  CHECK(check_ptr(k, fn, "k"));
  CHECK(check_ptr(v, fn, "v"));
  CHECK(check_ptr(out, fn, "out"));
  CHECK(check_ptr(ws, fn, "ws"));
  const size_t need = layer_bufs(a, topk, nullptr, nullptr);
  if (ws_bytes < need) return spark_set_error(SPARK_E_WORKSPACE, "%s: ws_bytes %zu < %zu", fn, ws_bytes, need);
  LayerBufs b;
  layer_bufs(a, topk, (char*)ws, &b);
  const size_t scratch_bytes = need - (size_t)((char*)b.scratch - (char*)ws);
  CHECK(spark_reblock(a, q, k, v, b.perm_q, b.perm_k, b.q_p, b.k_p, b.v_pt, b.qbar, b.kbar, b.anchor,
                      b.scratch, scratch_bytes, stream));
  CHECK(spark_select(a, b.qbar, b.kbar, nullptr, topk, b.idx, nullptr, stream));
  CHECK(spark_summarize(a, b.k_p, b.v_pt, b.anchor, b.ksum, b.vsum, b.bias, stream));
  return spark_attn(a, b.q_p, b.k_p, b.v_pt, b.idx, topk, b.ksum, b.vsum, b.bias, b.perm_q, out,
                    b.scratch, scratch_bytes, stream);
}

}  // extern "C"

int spark_diagnostics(const spark_args* a, const void* q_p, const void* k_p, const int32_t* idx,
                      int32_t topk, const float* ksum, const float* bias, float* recall,
                      float* logmass, spark_stream_t stream) {
  const char* fn = "spark_diagnostics";
  CHECK(check_args(a, fn));
  CHECK(reject_context(a, fn));
  if (fp8_of(a)) return spark_set_error(SPARK_E_UNSUPPORTED, "%s: SPARK_EXACT_FP8 is not supported here", fn);
  const int nb = nblocks(a);
  if (topk < 1 || topk > nb) return spark_set_error(SPARK_E_SHAPE, "%s: topk=%d not in [1, %d]", fn, topk, nb);
  CHECK(check_ptr(q_p, fn, "q_p"));
  CHECK(check_ptr(k_p, fn, "k_p"));
  CHECK(check_ptr(idx, fn, "idx"));
  CHECK(check_ptr(ksum, fn, "ksum"));
  CHECK(check_ptr(bias, fn, "bias"));
  CHECK(check_ptr(recall, fn, "recall", true));
  CHECK(check_ptr(logmass, fn, "logmass", true));
  if (recall == nullptr && logmass == nullptr)
    return spark_set_error(SPARK_E_ARG, "%s: recall and logmass are both NULL", fn);
  return diag_launch(a->H, a->N, a->d, a->block, a->dtype, q_p, k_p, idx, topk, ksum, bias, recall, logmass, (hipStream_t)stream);
}

int spark_quant_e4m3(int32_t rows, int32_t d, int32_t group, int32_t dtype, const void* x, uint8_t* x8,
                     float* scales, spark_stream_t stream) {
  const char* fn = "spark_quant_e4m3";
  if (rows < 1 || group < 1) return spark_set_error(SPARK_E_SHAPE, "%s: rows=%d group=%d", fn, rows, group);
  if (d != 64 && d != 128) return spark_set_error(SPARK_E_UNSUPPORTED, "%s: d=%d not in {64, 128}", fn, d);
  if (dtype != SPARK_F32 && dtype != SPARK_BF16)
    return spark_set_error(SPARK_E_DTYPE, "%s: dtype %d is not SPARK_F32/SPARK_BF16", fn, dtype);
  CHECK(check_ptr(x, fn, "x"));
  if (x8 == nullptr || scales == nullptr) return spark_set_error(SPARK_E_ARG, "%s: x8 or scales is NULL", fn);
  if (reinterpret_cast<uintptr_t>(x8) % 4 != 0)
    return spark_set_error(SPARK_E_ARG, "%s: x8 is not 4-byte aligned", fn);
  return quant_e4m3_launch(1, rows, rows, d, group, dtype, x, x8, scales, (hipStream_t)stream);
}

// ---- test hooks ---------------------------------------------------------------------
size_t spark_debug_partition_ws_bytes(int32_t count, int32_t n, int32_t block) {
  if (count < 1 || n < 1 || block < 1 || block > 128 || (long)count * n > 0x7fffffffL) {
    spark_set_error(SPARK_E_SHAPE, "spark_debug_partition_ws_bytes: count=%d n=%d block=%d", count, n, block);
    return (size_t)-1;
  }
  return debug_partition_ws_bytes(count, n, block);
}

int spark_debug_partition_level(int32_t count, int32_t n, int32_t block, const float* s,
                                const int32_t* ids_in, int32_t* ids_out, void* ws, size_t ws_bytes,
                                spark_stream_t stream) {
  const char* fn = "spark_debug_partition_level";
  if (count < 1 || n < 1 || block < 1 || block > 128 || (long)count * n > 0x7fffffffL)
    return spark_set_error(SPARK_E_SHAPE, "%s: count=%d n=%d block=%d", fn, count, n, block);
  CHECK(check_ptr(s, fn, "s"));
  CHECK(check_ptr(ids_in, fn, "ids_in"));
  CHECK(check_ptr(ids_out, fn, "ids_out"));
  const size_t need = debug_partition_ws_bytes(count, n, block);
  CHECK(check_ptr(ws, fn, "ws"));
  if (ws_bytes < need) return spark_set_error(SPARK_E_WORKSPACE, "%s: ws_bytes %zu < %zu", fn, ws_bytes, need);
  return debug_partition_launch(count, n, block, s, ids_in, ids_out, ws, (hipStream_t)stream);
}

int spark_debug_argmin(int32_t count, int32_t n, const float* vals, const int32_t* ids, int32_t* out,
                       spark_stream_t stream) {
  const char* fn = "spark_debug_argmin";
  if (count < 1 || n < 1 || (long)count * n > 0x7fffffffL)
    return spark_set_error(SPARK_E_SHAPE, "%s: count=%d n=%d", fn, count, n);
  CHECK(check_ptr(vals, fn, "vals"));
  CHECK(check_ptr(ids, fn, "ids"));
  CHECK(check_ptr(out, fn, "out"));
  return debug_argmin_launch(count, n, vals, ids, out, (hipStream_t)stream);
}

// ---- measurement helper ---------------------------------------------------------------
double spark_mfma_peak_probe(int32_t workgroups, int32_t iters, float* sink, spark_stream_t stream) {
  if (workgroups < 1 || iters < 1) {
    spark_set_error(SPARK_E_SHAPE, "spark_mfma_peak_probe: workgroups=%d iters=%d", workgroups, iters);
    return -1.0;
  }
  if (check_ptr(sink, "spark_mfma_peak_probe", "sink")) return -1.0;
  if (mfma_peak_launch(workgroups, iters, sink, (hipStream_t)stream)) return -1.0;
  return (double)workgroups * 4 * 4 * (double)iters * (32.0 * 32.0 * 16.0 * 2.0);
}
