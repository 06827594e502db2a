// HIP kernel of the non-absorbed MLA prefill, written for gfx950.
//
// In prefill the latent is decompressed into per-head K and V and a standard
// multi-head attention kernel runs over them ("MLA & DSA 推理性能优化指南"
// §3.1; the non-absorbed path of the §1.1 figure); per head the key is
// [W_UK c_t | k_rope_t] (128 + 64 dims, §5.1), the value W_UV c_t (128).
// Given those per-head Q, K, V this kernel computes, per (b, h, t),
//   out = sum_j softmax(scale q_t . k_j) v_j over j <= t (causal) or j < T,
//   lse = ln sum_j exp(scale q_t . k_j).
//
// One workgroup per (256 query rows, head, sequence); wave w owns rows
// 32w..32w+31 with their Q in registers.  K/V tiles of 64 tokens are staged in
// LDS by the whole workgroup (K row-padded, V stored transposed so that the
// P.V operand reads are contiguous).  Per tile and wave: S^T = K Q^T with bf16
// MFMA 32x32x16 over 192 dims, an online softmax in the log2 domain, P moved
// into the MFMA operand layout by lane swaps in registers, and O^T += V^T P^T
// (fp32 accumulation).  Tiles entirely above a wave's rows are
// skipped under the causal rule.
#include "mla_internal.h"

#include <utility>

namespace mla {
namespace kern {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDqk = 192, kDv = 128;
constexpr int kWaves = 8, kRowsWg = 32 * kWaves, kTile = 64;
constexpr int kKStride = 200;  // bf16 elements per K row in LDS (400 B, 16-byte aligned, padded)
constexpr int kVStride = 72;   // bf16 elements per V^T row (64 tokens + pad)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309f;

// K operand reads issued from assembly with explicit counted waits, so that
// several are in flight per MFMA (the compiler keeps about two).  At the
// start of a tile's scores no other LDS operation of the wave is pending
// (the workgroup barrier drained them), so the counts are exact.
template <int OFF>
__device__ __forceinline__ void lds_rd16(bf16x8& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "n"(OFF));
}
template <int N>
__device__ __forceinline__ void lds_ready(bf16x8& v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}
template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

__global__ __launch_bounds__(64 * kWaves, 1) void prefill_kernel(PrefillArgs a) {
  // three buffers: tile j + 1 is stored while tile j (scores) and tile
  // j - 1 (its P.V, pipelined into step j) are read
  __shared__ __attribute__((aligned(16))) __bf16 k_lds2[3][kTile * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds2[3][kDv * kVStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  // the last query tiles see the most keys: dispatch them first
  const int t0 = (gridDim.x - 1 - blockIdx.x) * kRowsWg;
  const int h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, H = a.H;
  const size_t seq = (size_t)b * T;
  const int row = t0 + 32 * wave + l32;  // this lane's query position
  const bool row_ok = row < T;

  // Q of the wave's rows (B operand: row l32, dims 16 ks + 8 g .. + 7)
  bf16x8 qf[kDqk / 16];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + ((seq + (row_ok ? row : 0)) * H + h) * kDqk + 8 * g);
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ks++) qf[ks] = row_ok ? qp[2 * ks] : bf16x8{};
  }
  f32x16 o[kDv / 32];
#pragma unroll
  for (int d = 0; d < kDv / 32; d++) o[d] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.scale * kLog2e;

  const int last = a.causal ? min(T - 1, t0 + kRowsWg - 1) : T - 1;
  const int n_tiles = last / kTile + 1;
  const int wave_last = t0 + 32 * wave + 31;  // highest row of the wave
  // Tile loads: K as 64 tokens x 24 pieces of 8 dims (3 per thread); V as
  // 16 pieces of 8 dims x 64 tokens, a thread taking two consecutive tokens
  // of one piece (2 per thread), so that the transposing LDS stores write
  // both tokens of a dim as one 4-byte word and consecutive lanes hit
  // consecutive banks.  Tile j + 1 is loaded into registers while tile j is
  // computed and stored into the other LDS buffer afterwards: one workgroup
  // barrier per tile.
  constexpr int kThreads = 64 * kWaves;
  constexpr int kKPer = kTile * (kDqk / 8) / kThreads, kVPer = 2;
  static_assert(kTile * (kDv / 8) == kVPer * kThreads, "V tile split");
  bf16x8 kr[kKPer], vr[kVPer];
  const int v_tok = 2 * (tid % 32), v_pc = tid / 32;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kKPer; i++) {
      const int p = tid + kThreads * i, tok = p / (kDqk / 8), pc = p % (kDqk / 8);
      kr[i] = k0 + tok < T ? *reinterpret_cast<const bf16x8*>(a.k + ((seq + k0 + tok) * H + h) * kDqk + 8 * pc)
                           : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < kVPer; i++) {
      const int tok = v_tok + i;
      vr[i] = k0 + tok < T ? *reinterpret_cast<const bf16x8*>(a.v + ((seq + k0 + tok) * H + h) * kDv + 8 * v_pc)
                           : bf16x8{};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKPer; i++) {
      const int p = tid + kThreads * i, tok = p / (kDqk / 8), pc = p % (kDqk / 8);
      *reinterpret_cast<bf16x8*>(&k_lds2[buf][tok * kKStride + 8 * pc]) = kr[i];
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
      bf16x2 w = {vr[0][e], vr[1][e]};
      *reinterpret_cast<bf16x2*>(&vt_lds2[buf][(8 * v_pc + e) * kVStride + v_tok]) = w;
    }
  };
  // P.V of tile j - 1 runs in step j beside tile j's softmax.  Before the
  // first tile it runs on a zeroed V buffer with P = 0 (adds nothing), so
  // the common step has no branch between the two.
  bf16x8 pf_prev[kTile / 16];
#pragma unroll
  for (int kk = 0; kk < kTile / 16; kk++) pf_prev[kk] = bf16x8{};
  float alpha_prev = 1.f;
  bool pend = false;
  for (int i = tid; i < kDv * kVStride / 2; i += kThreads) reinterpret_cast<unsigned*>(vt_lds2[2])[i] = 0u;
  auto pv_step = [&](const __bf16* vt) {
#pragma unroll
    for (int kk = 0; kk < kTile / 16; kk++) {
#pragma unroll
      for (int d = 0; d < kDv / 32; d++) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vt[(32 * d + l32) * kVStride + 16 * kk + 8 * g]);
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf_prev[kk], o[d], 0, 0, 0);
      }
    }
  };
  auto rescale_prev = [&]() {  // O only needs rescaling when some row's maximum moved
    if (__builtin_amdgcn_ballot_w64(alpha_prev != 1.f) != 0) {
#pragma unroll
      for (int d = 0; d < kDv / 32; d++) o[d] *= alpha_prev;
    }
  };
  load_tile(0);
  store_tile(0);
  __syncthreads();
  int cur = 0;  // buffer of tile j; tile j - 1 is in (cur + 2) % 3
  for (int j = 0; j < n_tiles; j++) {
    const int k0 = j * kTile;
    const int prv = cur == 0 ? 2 : cur - 1, nxt = cur == 2 ? 0 : cur + 1;
    const __bf16* k_lds = k_lds2[cur];
    const bool more = j + 1 < n_tiles;
    if (more) load_tile(k0 + kTile);
    if (a.causal && k0 > wave_last) {
      // the whole tile lies above this wave's rows: only finish the last
      // computed tile's P.V (once)
      if (pend) {
        rescale_prev();
        pv_step(vt_lds2[prv]);
        pend = false;
      }
    } else {

    // S^T[token][row] = K Q^T over 192 dims for the tile's two 32-token
    // halves; lane holds row l32 and tokens 32 hf + 8 (i / 4) + 4 g + i % 4
    // operand n = 2 ks + hf: token 32 hf + l32, dims 16 ks + 8 g .. + 7
    f32x16 s2[2] = {f32x16{}, f32x16{}};
    {
      constexpr int kN = 2 * (kDqk / 16), kLead = 4, kRing = 6;
      const uint32_t kb = (uint32_t)reinterpret_cast<uintptr_t>(k_lds);
      const uint32_t ad[2] = {kb + (uint32_t)((l32 * kKStride + 8 * g) * 2),
                              kb + (uint32_t)(((32 + l32) * kKStride + 8 * g) * 2)};
      bf16x8 ring[kRing];
      auto rd = [&](auto NI) {
        constexpr int n = decltype(NI)::value;
        lds_rd16<32 * (n / 2)>(ring[n % kRing], ad[n % 2]);
      };
      unroll<kLead>(rd);
      unroll<kN>([&](auto NI) {
        constexpr int n = decltype(NI)::value;
        lds_ready<(kLead - 1 < kN - 1 - n ? kLead - 1 : kN - 1 - n)>(ring[n % kRing]);
        s2[n % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % kRing], qf[n / 2], s2[n % 2], 0, 0, 0);
        if constexpr (n + kLead < kN) rd(std::integral_constant<int, n + kLead>{});
      });
    }
    // rescale O for tile j - 1's maximum before its P.V (a branch, kept out
    // of the block where that P.V interleaves with this tile's softmax)
    rescale_prev();
    // mask (only tiles that reach past T or above the wave's first row need
    // it), then the online softmax (max over unscaled scores: scale > 0)
    float mloc = kNegInf;
    const bool full = k0 + kTile <= T && (!a.causal || k0 + kTile - 1 <= t0 + 32 * wave) && t0 + 32 * wave + 31 < T;
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; i++) mloc = fmaxf(mloc, s2[hf][i]);
      } else {
        // the row sees tokens up to lim (none when the row is past T);
        // token k0 + 32 hf + 8 (i / 4) + 4 g + i % 4 against it
        const int lim = (row_ok ? (a.causal ? min(row, T - 1) : T - 1) : -1) - (k0 + 32 * hf + 4 * g);
#pragma unroll
        for (int i = 0; i < 16; i++) {
          s2[hf][i] = 8 * (i / 4) + (i % 4) <= lim ? s2[hf][i] : kNegInf;
          mloc = fmaxf(mloc, s2[hf][i]);
        }
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc * c2);
    const float muse = m_new == kNegInf ? 0.f : m_new;
    const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run - muse);
    m_run = m_new;
    // P in the operand layout of O^T += V^T P^T without a trip through LDS:
    // for tokens 16 kk .. 16 kk + 15 lane (l32, g) holds, per half g, 4 of
    // the 8 tokens its operand needs; swapping the second group of the lower
    // lanes with the first group of the upper lanes (v_permlane32_swap)
    // gives every lane its 8 consecutive tokens 16 kk + 8 g .. + 7.
    float psum = 0.f;
    bf16x8 pf[kTile / 16];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        // a masked score is -inf, and exp2(-inf) = 0 (muse is finite)
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[hf][i], c2, -muse));
        psum += pv[i];
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++) {  // tokens 32 hf + 16 h2 .. + 15
        unsigned xw[2], yw[2];
#pragma unroll
        for (int e = 0; e < 2; e++) {
          bf16x2 xa = {(__bf16)pv[8 * h2 + 2 * e], (__bf16)pv[8 * h2 + 2 * e + 1]};
          bf16x2 ya = {(__bf16)pv[8 * h2 + 4 + 2 * e], (__bf16)pv[8 * h2 + 4 + 2 * e + 1]};
          const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, xa),
                                                          __builtin_bit_cast(unsigned, ya), false, false);
          xw[e] = r[0];
          yw[e] = r[1];
        }
        u32x4 w = {xw[0], xw[1], yw[0], yw[1]};
        pf[2 * hf + h2] = __builtin_bit_cast(bf16x8, w);
      }
    }
    l_run = l_run * alpha + psum;
    pv_step(vt_lds2[prv]);  // tile j - 1 (or nothing before the first tile)
#pragma unroll
    for (int kk = 0; kk < kTile / 16; kk++) pf_prev[kk] = pf[kk];
    alpha_prev = alpha;
    pend = true;
    }
    // tile j + 1 goes to the buffer that tile j - 2 used: last read before
    // the previous barrier
    if (more) store_tile(nxt);
    __syncthreads();
    cur = nxt;
  }
  if (pend) {
    rescale_prev();
    pv_step(vt_lds2[cur == 0 ? 2 : cur - 1]);
  }

  // O^T[dim][row]: lane holds row l32, dims 32 d + 8 (i / 4) + 4 g + i % 4
  const float l = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  __bf16* op = reinterpret_cast<__bf16*>(a.out) + ((seq + row) * H + h) * kDv + 4 * g;
#pragma unroll
  for (int d = 0; d < kDv / 32; d++) {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      bf16x4 w = {(__bf16)(o[d][4 * q4] * inv), (__bf16)(o[d][4 * q4 + 1] * inv),
                  (__bf16)(o[d][4 * q4 + 2] * inv), (__bf16)(o[d][4 * q4 + 3] * inv)};
      *reinterpret_cast<bf16x4*>(op + 32 * d + 8 * q4) = w;
    }
  }
  if (g == 0) a.lse[(seq + row) * H + h] = empty ? kNegInf : (m_run + __log2f(l)) * kLn2;
}

}  // namespace
}  // namespace kern

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.T + kern::kRowsWg - 1) / kern::kRowsWg), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(kern::prefill_kernel, grid, dim3(64 * kern::kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
