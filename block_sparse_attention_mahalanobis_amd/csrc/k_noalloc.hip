// Allocation-free form of spark_attn for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation).  Its scratch -- the bf16 summary tiles and the
// log2-domain bias the attention kernels stream, and for E4M3 logits the
// quantised keys -- lives in one file-scope device array of fixed size
// instead of a caller workspace.  Each GPU the library runs on holds its own
// copy of the array until the process ends.
//
// The host never uses the array's name as an address (on the host it is only
// a stand-in symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device.
//
// Every call on one GPU shares that GPU's array and leaves its last contents
// there; calls that overlap on one GPU (two streams, or two host threads)
// race on it and must be serialised by the caller.  Nothing in the array has
// to start at zero: the summary pass rewrites every byte the attention
// kernels read (padding blocks included) before they run.
#include <mutex>

#include "common.hpp"

namespace spark {

int attn_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* qp, const void* kp,
                const void* vpt, const int32_t* idx, int topk, const float* ksum,
                const float* vsum, const float* bias, const int32_t* perm_q, void* out, void* ws,
                bool fp8, bool paired, hipStream_t st);

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;   // 64 MiB per GPU
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];

size_t noalloc_scratch_bytes() { return NOALLOC_SCRATCH_BYTES; }

// Device address of the current device's copy of `scratch` (looked up on the
// first call made with that device current).
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return spark_set_error(SPARK_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return spark_set_error(SPARK_E_HIP, "device %d outside the %d devices the scratch table holds", dev,
                           NOALLOC_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return spark_set_error(SPARK_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                             hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPARK_OK;
}

// The caller has validated the arguments and checked that the workspace
// spark_attn would need fits NOALLOC_SCRATCH_BYTES.
int attn_noalloc_launch(int H, int N, int Nv, int D, int BK, int dtype, const void* qp, const void* kp,
                        const void* vpt, const int32_t* idx, int topk, const float* ksum,
                        const float* vsum, const float* bias, const int32_t* perm_q, void* out,
                        bool fp8, bool paired, hipStream_t st) {
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return attn_launch(H, N, Nv, D, BK, dtype, qp, kp, vpt, idx, topk, ksum, vsum, bias, perm_q, out, ws,
                     fp8, paired, st);
}

}  // namespace spark
