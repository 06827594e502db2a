// The per-head GEMM of the projections around the absorbed decode, as a
// device function of one 256-thread workgroup (see mla_proj.hip), so that
// other launches can run it beside their own work.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace kern {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// K: contraction length, N: output columns per head, SPLIT: waves that
// share one 32-column tile, each taking 1/SPLIT of the contraction (their
// partial tiles are summed through LDS).  A workgroup of 4 waves computes
// 4/SPLIT tiles of 32 columns of one head for a block of rows.  The long
// contraction (K = 512) is split 4 ways.
template <int K, int N, int SPLIT>
struct ProjTile {
  static constexpr int kCols = 32 * 4 / SPLIT;      // columns per workgroup
  static constexpr int kRows = SPLIT > 1 ? 64 : 128;  // rows per row block
  static constexpr int kRowBytes = 2 * K;           // one weight or activation row
  // With the contraction split over the waves, each wave reads its weight
  // fragment once: it loads it from HBM into registers, and only the
  // activation tile is staged (so two workgroups fit on a CU).
  static constexpr bool kWDirect = SPLIT > 1;
  static constexpr int kWBytes = kWDirect ? 0 : kCols * kRowBytes;  // the weight tile in LDS
  static constexpr int kABytes = kRows * kRowBytes; // the activation tile
  static constexpr int kRedOff = kWBytes + kABytes; // partial tiles of the non-leading waves
  static constexpr int kLdsBytes = kRedOff + (SPLIT > 1 ? 3 * 16 * 64 * 4 : 0);
  static constexpr int kCopies = (kWBytes + kABytes) / 1024;
  static_assert(kRowBytes <= 1024 && 1024 % kRowBytes == 0 && kCopies % 4 == 0, "copy shape");
  static_assert(kLdsBytes <= 80 * 1024, "LDS budget: two workgroups per CU");
};

// The activation tile (and, without a split contraction, the weight tile)
// is staged in LDS by direct copies of whole rows (1 KB per copy: a weight
// or activation row is 256 B or 1 KB, contiguous in HBM), so every such
// HBM read is fully coalesced; 16-byte chunk c of tile row r sits at
// position c ^ (r & 15), so that the MFMA operand reads (one chunk of 16
// consecutive rows per 16 lanes) cover every bank.  `lds` is the dynamic
// LDS of the launch, ProjTile<K, N, SPLIT>::kLdsBytes bytes.
template <int K, int N, int SPLIT>
__device__ __forceinline__ void head_gemm(const ProjArgs& a, uint8_t* lds, int bx, int h, int bz) {
  using T = ProjTile<K, N, SPLIT>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int H = a.H, M = a.M;
  const int n_base = bx * T::kCols, m_base = bz * T::kRows;
  constexpr int kChunks = K / 8, kRowsPerCopy = 1024 / T::kRowBytes;
  const int part = wave % SPLIT;               // which share of the contraction
  const int col0 = (wave / SPLIT) * 32;        // the wave's columns within the tile
  constexpr int KS = K / SPLIT / 16;           // k-steps per wave
  const int kc0 = part * (K / SPLIT / 8);      // first chunk of the wave's share
  const int wr = col0 + l32;                   // weight tile row of this lane
  bf16x8 wf[KS];
  if constexpr (T::kWDirect) {
    const bf16x8* wp = reinterpret_cast<const bf16x8*>(a.w + ((size_t)h * N + n_base + wr) * K) + kc0 + g;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) wf[ks] = wp[2 * ks];
  }
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int rr = ln / kChunks, p = ln % kChunks;  // row within the copy, LDS chunk position
#pragma unroll
    for (int i = 0; i < T::kCopies / 4; i++) {
      const int cpy = 4 * i + wave;
      const uint8_t* src;
      int row;
      if (cpy < T::kWBytes / 1024) {
        row = cpy * kRowsPerCopy + rr;
        src = reinterpret_cast<const uint8_t*>(a.w + ((size_t)h * N + n_base + row) * K);
      } else {
        const int r0 = (cpy - T::kWBytes / 1024) * kRowsPerCopy;
        if (m_base + r0 >= M) continue;  // (wave-uniform) rows past M are never read
        row = r0 + rr;
        const int m = min(m_base + row, M - 1);  // rows past M are never stored
        src = reinterpret_cast<const uint8_t*>(a.a + ((size_t)m * H + h) * K);
      }
      copy16_v(src + ((p ^ (row & 15)) << 4), lds_addr(lds + cpy * 1024));
    }
  }
  wait_vm<0>();
  __syncthreads();

  if constexpr (!T::kWDirect) {
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      wf[ks] = *reinterpret_cast<const bf16x8*>(lds + wr * T::kRowBytes + (((kc0 + 2 * ks + g) ^ (wr & 15)) << 4));
  }
  float* const red = reinterpret_cast<float*>(lds + T::kRedOff);
#pragma unroll
  for (int mt = 0; mt < T::kRows / 32; mt++) {
    const int m0 = m_base + 32 * mt;
    if (m0 >= M) break;  // uniform over the workgroup
    const int ar = 32 * mt + l32;              // activation tile row of this lane
    const int row = m0 + l32;
    const bool ok = row < M;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(lds + T::kWBytes + ar * T::kRowBytes +
                                                         (((kc0 + 2 * ks + g) ^ (ar & 15)) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], af, acc, 0, 0, 0);
    }
    if constexpr (SPLIT > 1) {
      if (part > 0) {
#pragma unroll
        for (int r = 0; r < 16; r++) red[((part - 1) * 16 + r) * 64 + lane] = acc[r];
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int r = 0; r < 16; r++)
          acc[r] += red[r * 64 + lane] + red[(16 + r) * 64 + lane] + red[(32 + r) * 64 + lane];
      }
    }
    // lane holds column m = row, rows n = n_base + col0 + 8 q + 4 g + i (i < 4) of D^T
    if (part == 0 && ok) {
      __bf16* crow = reinterpret_cast<__bf16*>(a.c) + ((size_t)row * H + h) * N + n_base + col0 + 4 * g;
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
