// Dense decode for callers that cannot allocate device memory: the split
// workspace is a fixed device array of this library instead of a buffer the
// caller passes in.  Everything else is mla_decode: the same validation, the
// same kernels, the same results.
#include <mutex>

#include "mla.h"
#include "mla_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;

// The workspace of mla_decode_noalloc.  Host code never uses this name as an
// address (on the host it is only a handle for the symbol lookup below);
// kernels get the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current; nullptr (and *err set) on failure.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || p == nullptr) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const void* q_nope, const void* q_rope,
                                         const void* kv_pages, const float* kv_scales,
                                         mla_kv_dtype kv_dtype, int num_pages,
                                         const int32_t* block_table, int bt_stride,
                                         const int32_t* cache_seqlens, int B, int Sq, int H,
                                         float softmax_scale, int causal, void* out, float* lse,
                                         int num_wg, hipStream_t stream) {
  const size_t need = mla_workspace_size(B, Sq, H, 0, num_wg);
  if (need == 0) return mla::fail_status(MLA_ERR_SHAPE, "sizes out of range");
  if (need > kScratchBytes)
    return mla::fail_status(MLA_ERR_WORKSPACE,
                            "these sizes need more workspace than the static scratch of "
                            "mla_decode_noalloc holds (MLA_NOALLOC_SCRATCH_BYTES)");
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (ws == nullptr) return mla::fail_status(MLA_ERR_HIP, hipGetErrorString(e));
  // The scheduling pass rewrites every workspace entry the later stages
  // read, so nothing a previous call left there needs clearing.
  return mla::run_decode(q_nope, q_rope, kv_pages, kv_scales, kv_dtype, num_pages, block_table,
                         bt_stride, cache_seqlens, nullptr, 0, B, Sq, H, softmax_scale, causal, out,
                         lse, ws, kScratchBytes, num_wg, 0, stream);
}
