// The absorbed decode layer, for gfx950.
//
// "MLA 最佳算子全景调研" §2 credits a fused decode kernel's gain to doing the
// query absorption, the attention and the output projection together; around
// the latent-space decode ("MLA & DSA 推理性能优化指南" §1.1 figure, §5.1) the
// layer is
//   q_nope[m, h, :] = q_c[m, h, :] . W_UK[h]          (128 -> 512, per head)
//   out, lse        = absorbed decode over the latent cache
//   o[m, h, :]      = W_UV[h] . out[m, h, :]           (512 -> 128, per head)
// One op at a time it is four launches: absorb, main pass (computing its
// own split-KV schedule first), split merge, projection.  The schedule only
// reads the sequence lengths, so here it runs as one more workgroup of the
// absorption launch (absorb_plan_kernel), beside the GEMM, and the main
// pass reads its share instead of computing it.  The other
// steps stay separate launches on purpose: the absorption and the
// projection read each head's weights once only when a workgroup covers the
// rows of one head over the whole batch, while the main pass and the split
// merge are organised by sequence (one sequence's rows are all heads), and
// the split partials are stored in the order the main pass's accumulators
// leave the registers -- 128-byte lines that interleave eight heads.  A
// merge organised by head, to feed the projection without a trip through
// HBM, reads every line eight times; on a 64-sequence, 128-head batch it ran
// several times slower than the merge by sequence plus the projection.
#include "mla_device.h"
#include "mla_internal.h"
#include "mla_proj.h"
#include "mla_sched.h"

namespace mla {
namespace kern {

// Grid: one scheduling workgroup (block 0), then 4 x H x ceil(M / 128)
// absorption workgroups (128 columns, head, row block of 128).
__global__ __launch_bounds__(256) void absorb_plan_kernel(LayerArgs la) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int i = blockIdx.x;
  if (i == 0) {
    plan_work<false>(la.d);
    return;
  }
  // the GEMM's workgroups of one head on one XCD (see head_gemm_kernel)
  const int j = xcd_logical(i - 1, gridDim.x - 1);
  const int H = la.pa.H;
  head_gemm<kDHead, kDC, 1>(la.pa, lds, j & 3, (j >> 2) % H, (j >> 2) / H);
}

}  // namespace kern

hipError_t launch_absorb_plan(const LayerArgs& la, hipStream_t stream) {
  using T = kern::ProjTile<kDHead, kDC, 1>;
  static_assert(kDC / T::kCols == 4, "four column tiles per head");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern::absorb_plan_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, T::kLdsBytes);
  if (e != hipSuccess) return e;
  const long long mblocks = (la.pa.M + T::kRows - 1) / T::kRows;
  const long long grid = 1 + 4LL * la.pa.H * mblocks;
  hipLaunchKernelGGL(kern::absorb_plan_kernel, dim3((unsigned)grid), dim3(256), T::kLdsBytes, stream, la);
  return hipGetLastError();
}

}  // namespace mla
