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
#include "mla_internal.h"

namespace mla {
namespace kern {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowsPerBlock = 128;

// K: contraction length, N: output columns per head, SPLIT: waves that
// share one 32-column tile, each taking 1/SPLIT of the contraction (their
// partial tiles are summed through LDS).  A workgroup of 4 waves computes
// 4/SPLIT tiles of 32 columns of one head for up to 128 rows.  The long
// contraction (K = 512) is split 4 ways: four times the waves of one wave
// per tile, and a quarter of the dependent load chain per wave.
template <int K, int N, int SPLIT>
__global__ __launch_bounds__(256) void head_gemm_kernel(ProjArgs a) {
  __shared__ float red[SPLIT > 1 ? 3 : 1][16][64];  // partial tiles of the non-leading waves
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int part = wave % SPLIT;               // which share of the contraction
  const int n0 = (blockIdx.x * (4 / SPLIT) + wave / SPLIT) * 32;
  const int h = blockIdx.y;
  const int m_base = blockIdx.z * kRowsPerBlock;
  const int H = a.H, M = a.M;
  constexpr int KW = K / SPLIT;
  constexpr int KS = KW / 16;
  const int k_off = part * KW;
  // weight fragments: row n0 + l32 of Bt[h], k = k_off + 16 ks + 8 g .. + 7
  bf16x8 wf[KS];
  const bf16x8* wrow = reinterpret_cast<const bf16x8*>(a.w + ((size_t)h * N + n0 + l32) * K + k_off + 8 * g);
#pragma unroll
  for (int ks = 0; ks < KS; ks++) wf[ks] = wrow[2 * ks];
  // every row tile's activations are requested together with the weights:
  // one memory round trip for the whole workgroup
  constexpr int kMT = kRowsPerBlock / 32;
  bf16x8 av_all[kMT][KS];
#pragma unroll
  for (int mt = 0; mt < kMT; mt++) {
    const int m0 = m_base + 32 * mt;
    const int row = m0 + l32;
    const bool ok = m0 < M && row < M;
    const bf16x8* arow =
        reinterpret_cast<const bf16x8*>(a.a + ((size_t)(ok ? row : 0) * H + h) * K + k_off + 8 * g);
#pragma unroll
    for (int ks = 0; ks < KS; ks++) av_all[mt][ks] = ok ? arow[2 * ks] : bf16x8{};
  }
#pragma unroll
  for (int mt = 0; mt < kMT; mt++) {
    const int m0 = m_base + 32 * mt;
    if (m0 >= M) break;  // uniform over the workgroup
    const int row = m0 + l32;
    const bool ok = row < M;
    const bf16x8* av = av_all[mt];
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ks++) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], av[ks], acc, 0, 0, 0);
    if constexpr (SPLIT > 1) {
      if (part > 0) {
#pragma unroll
        for (int r = 0; r < 16; r++) red[part - 1][r][lane] = acc[r];
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int r = 0; r < 16; r++) acc[r] += red[0][r][lane] + red[1][r][lane] + red[2][r][lane];
      }
    }
    // lane holds column m = row, rows n = n0 + 8 q + 4 g + i (i < 4) of D^T
    if (part == 0 && ok) {
      __bf16* crow = reinterpret_cast<__bf16*>(a.c) + ((size_t)row * H + h) * N + n0 + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        bf16x4 v = {(__bf16)acc[4 * q], (__bf16)acc[4 * q + 1], (__bf16)acc[4 * q + 2], (__bf16)acc[4 * q + 3]};
        *reinterpret_cast<bf16x4*>(crow + 8 * q) = v;
      }
    }
    if constexpr (SPLIT > 1) __syncthreads();
  }
}

}  // namespace
}  // namespace kern

hipError_t launch_proj(const ProjArgs& a, bool absorb, hipStream_t stream) {
  const unsigned mblocks = (unsigned)((a.M + kern::kRowsPerBlock - 1) / kern::kRowsPerBlock);
  if (absorb)  // K = 128, N = 512
    hipLaunchKernelGGL((kern::head_gemm_kernel<kDHead, kDC, 1>), dim3(kDC / 128, a.H, mblocks), dim3(256),
                       0, stream, a);
  else         // K = 512, N = 128
    hipLaunchKernelGGL((kern::head_gemm_kernel<kDC, kDHead, 4>), dim3(kDHead / 32, a.H, mblocks), dim3(256),
                       0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
