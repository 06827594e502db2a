// The per-head GEMM of the projections around the absorbed decode, as a
// device function of one 256-thread workgroup (see mla_proj.hip), so that
// other launches can run it beside their own work.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace kern {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 128;

// K: contraction length, N: output columns per head, SPLIT: waves that
// share one 32-column tile, each taking 1/SPLIT of the contraction (their
// partial tiles are summed through LDS).  A workgroup of 4 waves computes
// 4/SPLIT tiles of 32 columns of one head for up to 128 rows.  The long
// contraction (K = 512) is split 4 ways: four times the waves of one wave
// per tile, and a quarter of the dependent load chain per wave.
template <int K, int N, int SPLIT>
__device__ __forceinline__ void head_gemm(const ProjArgs& a, int bx, int h, int bz) {
  __shared__ float red[SPLIT > 1 ? 3 : 1][16][64];  // partial tiles of the non-leading waves
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int part = wave % SPLIT;               // which share of the contraction
  const int n0 = (bx * (4 / SPLIT) + wave / SPLIT) * 32;
  const int m_base = bz * kRowsPerBlock;
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

}  // namespace kern
}  // namespace mla
