// HIP kernels of the two per-head projections on either side of the
// absorbed decode, written for gfx950.
//
// With W_UK absorbed into the query ("MLA 在极长上下文下的显存带宽突围",
// section on absorbing the matrices at run time: q~ = q^C W^UK) the decode
// attends in the 512-dim latent space, and its 512-dim output per head is
// brought back to the head dimension by W_UV ("MLA & DSA 推理性能优化指南"
// §1.1 figure: W_UK and W_UV map d_c to d_h x n_h; §5.1: d_c = 512,
// d_h = 128, 128 heads):
//   absorb:  q_nope[m, h, :]  = q_c[m, h, :] . W_UK[h]         (128 -> 512)
//   project: o[m, h, :]       = W_UV[h] . out_latent[m, h, :]   (512 -> 128)
// Both are, per head, C[m][n] = sum_k A[m][k] Bt[n][k] with the contraction
// index contiguous in both operands: W_UK is kept as its transpose
// [H, 512, 128] (a storage choice made once for static weights), W_UV as
// [H, 128, 512].  A workgroup computes D^T = Bt A^T for 32 columns n of one
// head over up to 128 rows m with bf16 MFMA 32x32x16 and fp32 accumulation;
// its weight fragments stay in registers while it walks the row tiles, so
// every weight byte is read from HBM once.
#include "mla_device.h"
#include "mla_internal.h"
#include "mla_proj.h"

namespace mla {
namespace kern {
namespace {

// One workgroup per (column tile group, head, row block) on a flat grid;
// the workgroups of one head are consecutive logical workgroups of one XCD,
// so the activation rows that all of them read meet in that XCD's L2.
template <int K, int N, int SPLIT>
__global__ __launch_bounds__(256) void head_gemm_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NX = N / ProjTile<K, N, SPLIT>::kCols;  // column tiles per head
  const int lid = xcd_logical(blockIdx.x, gridDim.x);
  head_gemm<K, N, SPLIT>(a, lds, lid % NX, (lid / NX) % a.H, lid / (NX * a.H));
}

template <int K, int N, int SPLIT>
hipError_t launch_head_gemm(const ProjArgs& a, hipStream_t stream) {
  using T = ProjTile<K, N, SPLIT>;
  const void* f = reinterpret_cast<const void*>(head_gemm_kernel<K, N, SPLIT>);
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, T::kLdsBytes);
  if (e != hipSuccess) return e;
  const long long mblocks = (a.M + T::kRows - 1) / T::kRows;
  hipLaunchKernelGGL((head_gemm_kernel<K, N, SPLIT>), dim3((unsigned)((N / T::kCols) * a.H * mblocks)), dim3(256),
                     T::kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace kern


hipError_t launch_proj(const ProjArgs& a, bool absorb, hipStream_t stream) {
  if (absorb) return kern::launch_head_gemm<kDHead, kDC, 1>(a, stream);  // K = 128, N = 512
  return kern::launch_head_gemm<kDC, kDHead, 4>(a, stream);            // K = 512, N = 128
}

}  // namespace mla
