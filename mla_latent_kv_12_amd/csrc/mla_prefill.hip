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
// 32w..32w+31 with their Q in registers.  K/V tiles of 64 tokens are copied
// HBM -> LDS by the whole workgroup with direct copies of whole rows (5 per
// wave and tile), two tiles ahead of their use, into rings of 3 (K) and 4
// (V) buffers; rows are XOR-swizzled in 16-byte chunks for the operand
// reads.  Per tile and wave: S^T = K Q^T with bf16 MFMA 32x32x16 over 192
// dims, an online softmax in the log2 domain, and O^T += V^T P^T (fp32
// accumulation), V^T read by the transposing LDS read so that each lane's
// softmax weights are already its P operand.  The P.V of tile j - 1 runs in
// step j beside tile j's softmax.  Tiles entirely above a wave's rows are
// skipped under the causal rule.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace kern {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kDqk = 192, kDv = 128;
constexpr int kWaves = 8, kRowsWg = 32 * kWaves, kTile = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kKRow = 2 * kDqk, kVRow = 2 * kDv;  // bytes per K / V row
constexpr int kKBuf = kTile * kKRow, kVBuf = kTile * kVRow;
constexpr int kNK = 3, kNV = 4;                   // ring buffers
constexpr int kVOff = kNK * kKBuf;
constexpr int kLdsBytes = kVOff + kNV * kVBuf;
constexpr int kKCopies = kKBuf / 1024, kVCopies = kVBuf / 1024;
constexpr int kPerWave = (kKCopies + kVCopies) / kWaves;  // copies per wave and tile
static_assert((kKCopies + kVCopies) % kWaves == 0 && kLdsBytes <= 160 * 1024, "tile shape");

// K row r: 16-byte chunk c at position c ^ ((r >> 1) & 7) (the 16 rows of an
// operand read then cover every bank: a 384-byte row shifts the banks by
// half a row).  V row r: chunk c at position c ^ sw16(r & 15), the layout the
// transposing read below expects.
__device__ __forceinline__ int ksw(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int sw16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__global__ __launch_bounds__(64 * kWaves, 1) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int T = a.T, H = a.H;
  // Flat grid, one level of query tiles per H * B workgroups, the last query
  // tiles (which see the most keys) dispatched first, so that the light
  // tiles fill in at the end.  Workgroup i runs on XCD i % 8, so with H a
  // multiple of 8 all query tiles of one head share an XCD and its K/V
  // tiles meet in that XCD's L2.
  const int hb_n = H * a.B;
  const int level = blockIdx.x / hb_n, hb = blockIdx.x - level * hb_n;
  const int t0 = ((T + kRowsWg - 1) / kRowsWg - 1 - level) * kRowsWg;
  const int h = hb % H, b = hb / H;
  const size_t seq = (size_t)b * T;
  const int row = t0 + 32 * wave + l32;  // this lane's query position
  const bool row_ok = row < T;
  const int last = a.causal ? min(T - 1, t0 + kRowsWg - 1) : T - 1;
  const int n_tiles = last / kTile + 1;
  const int wave_last = t0 + 32 * wave + 31;  // highest row of the wave

  // Copies of tile j: copy i of this wave is copy number wave + 8 i of the
  // tile, K copies (i < 3) first, then V.  They go through buffer resources
  // over this (sequence, head)'s rows, so a row past T reads zeros (the
  // hardware range check; the mask gives those tokens weight 0), and each
  // lane's offset within a tile is computed once: a tile adds one
  // wave-uniform offset.
  static_assert(kKCopies == 3 * kWaves && kVCopies == 2 * kWaves, "copy split");
  const uint32_t krow_b = (uint32_t)H * kKRow, vrow_b = (uint32_t)H * kDv * 2;
  const i32x4 krs = make_rsrc(a.k + (seq * H + h) * kDqk, (uint32_t)(T - 1) * krow_b + kKRow);
  const i32x4 vrs = make_rsrc(a.v + (seq * H + h) * kDv, (uint32_t)(T - 1) * vrow_b + kVRow);
  uint32_t coff[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; i++) {
    int c = wave + kWaves * i;
    if (i < 3) {
      const int q = 64 * c + lane, r = q / (kKRow / 16), p = q % (kKRow / 16);
      coff[i] = (uint32_t)r * krow_b + (uint32_t)((p ^ ksw(r)) << 4);
    } else {
      c -= kKCopies;
      const int q = 64 * c + lane, r = q / (kVRow / 16), p = q % (kVRow / 16);
      coff[i] = (uint32_t)r * vrow_b + (uint32_t)((p ^ sw16(r)) << 4);
    }
  }
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(lds) + 1024 * wave);
  auto issue_copy = [&](int j, auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    const uint32_t k0 = (uint32_t)(j * kTile);
    if constexpr (i < 3)
      copy16_bs(krs, coff[i], k0 * krow_b, lds_wave + (j % kNK) * kKBuf + i * kWaves * 1024);
    else
      copy16_bs(vrs, coff[i], k0 * vrow_b, lds_wave + kVOff + (j % kNV) * kVBuf + (i - 3) * kWaves * 1024);
  };
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    unroll<kPerWave>([&](auto I) { issue_copy(j, I); });
  };

  // P.V of tile j - 1 runs in step j; before the first tile it runs on a
  // zeroed V buffer (the one tile -1 maps to) with P = 0.
  {
    uint4* z = reinterpret_cast<uint4*>(lds + kVOff + ((kNV - 1) % kNV) * kVBuf);
    for (int i = tid; i < kVBuf / 16; i += 64 * kWaves) z[i] = uint4{0u, 0u, 0u, 0u};
  }
  issue_tile(0);
  // Q of the wave's rows (B operand: row l32, dims 16 ks + 8 g .. + 7),
  // taken delivery of here (with tile 0): a wait left to the compiler would
  // land in the loop and also wait for the copies in flight there
  bf16x8 qf[kDqk / 16];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + ((seq + (row_ok ? row : 0)) * H + h) * kDqk + 8 * g);
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ks++) qf[ks] = row_ok ? qp[2 * ks] : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ks++) asm volatile("" : "+v"(qf[ks]));
  }
  wait_vm<0>();
  if (n_tiles > 1) issue_tile(1);
  __syncthreads();  // tile 0 and the zeroed V buffer are in LDS

  f32x16 o[kDv / 32];
#pragma unroll
  for (int d = 0; d < kDv / 32; d++) o[d] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.scale * kLog2e;

  // K operand offsets of this lane: token 32 hf + l32, chunk 2 ks + g at
  // position (2 ks + g) ^ ksw(token) = 8 (ks >> 2) + ((2 (ks & 3) + g) ^ kx)
  const int kx = ksw(l32);
  uint32_t koff[4];
#pragma unroll
  for (int j = 0; j < 4; j++) koff[j] = (uint32_t)(l32 * kKRow + (((2 * j + g) ^ kx) << 4));
  // V^T operand reads (transposing): lane loads token 16 kk + row0 (+ 8),
  // 4 dims of chunk 4 db + w
  int lnv = lane;
  asm volatile("" : "+v"(lnv));
  const int G16v = lnv >> 4, i16v = lnv & 15;
  const int row0 = 4 * (G16v >> 1) + (i16v >> 2);
  const int wv = 2 * (G16v & 1) + ((i16v >> 1) & 1);
  const uint32_t vbase = (uint32_t)(row0 * kVRow + 8 * (i16v & 1));
  const int vy0 = wv ^ sw16(row0), vy1 = wv ^ sw16(row0 + 8);

  bf16x8 pf_prev[kTile / 16];
#pragma unroll
  for (int kk = 0; kk < kTile / 16; kk++) pf_prev[kk] = bf16x8{};
  float alpha_prev = 1.f;
  bool pend = false;
  auto pv_step = [&](int vb_idx) __attribute__((always_inline)) {
    const uint8_t* vt = lds + kVOff + vb_idx * kVBuf;
#pragma unroll
    for (int kk = 0; kk < kTile / 16; kk++) {
#pragma unroll
      for (int d = 0; d < kDv / 32; d++) {
        const uint8_t* p0 = vt + vbase + (16 * kk) * kVRow + (((4 * d) ^ vy0) << 4);
        const uint8_t* p1 = vt + vbase + (16 * kk + 8) * kVRow + (((4 * d) ^ vy1) << 4);
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p0));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p1));
        const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pf_prev[kk], o[d], 0, 0, 0);
      }
    }
  };
  auto rescale_prev = [&]() __attribute__((always_inline)) {  // only when some row's maximum moved
    if (__builtin_amdgcn_ballot_w64(alpha_prev != 1.f) != 0) {
#pragma unroll
      for (int d = 0; d < kDv / 32; d++) o[d] *= alpha_prev;
    }
  };

  for (int j = 0; j < n_tiles; j++) {
    const int k0 = j * kTile;
    const bool ahead = j + 2 < n_tiles;
    if (a.causal && k0 > wave_last) {
      if (ahead) issue_tile(j + 2);
      // the whole tile lies above this wave's rows: only finish the last
      // computed tile's P.V (once)
      if (pend) {
        rescale_prev();
        pv_step((j + kNV - 1) % kNV);
        pend = false;
      }
    } else {
    // S^T[token][row] = K Q^T over 192 dims for the tile's two 32-token
    // halves; lane holds row l32 and tokens 32 hf + 8 (i / 4) + 4 g + i % 4.
    // Tile j + 2's copies go out between the MFMAs (a copy issued right
    // after another stalls its wave far longer than one between MFMAs).
    f32x16 s2[2] = {f32x16{}, f32x16{}};
    {
      constexpr int kN = 2 * (kDqk / 16), kLead = 4, kRing = 6;
      const uint32_t kb = lds_addr(lds + (j % kNK) * kKBuf);
      uint32_t ad[4];
#pragma unroll
      for (int q = 0; q < 4; q++) ad[q] = kb + koff[q];
      bf16x8 ring[kRing];
      // operand n = 2 ks + hf
      auto rd = [&](auto NI) {
        constexpr int n = decltype(NI)::value, ks = n / 2, hf = n % 2;
        lds_rd16<128 * (ks >> 2) + 32 * kKRow * hf>(ring[n % kRing], ad[ks & 3]);
      };
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the counted waits below start from zero
      unroll<kLead>(rd);
      unroll<kN>([&](auto NI) {
        constexpr int n = decltype(NI)::value;
        lds_ready<(kLead - 1 < kN - 1 - n ? kLead - 1 : kN - 1 - n)>(ring[n % kRing]);
        s2[n % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % kRing], qf[n / 2], s2[n % 2], 0, 0, 0);
        if constexpr (n % 5 == 2 && n / 5 < kPerWave) {
          if (ahead) issue_copy(j + 2, std::integral_constant<int, n / 5>{});
        }
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
    // The running maximum moves only when the tile exceeds it by more than
    // kRescaleSlack (log2 units), so O is rarely rescaled; weights stay
    // below 2^kRescaleSlack.  Before the row's first visible token O and l
    // are zero and need no factor.
    const float mc = mloc * c2;
    const bool need = mc > m_run + kRescaleSlack;  // -inf + slack = -inf
    const float alpha = need && m_run != kNegInf ? __builtin_amdgcn_exp2f(m_run - mc) : 1.f;
    if (need) m_run = mc;
    const float muse = m_run == kNegInf ? 0.f : m_run;
    // The weights are the P operand as they are: for k-step 2 hf + kk the
    // transposing V read pairs operand element e with token
    // 32 hf + 16 kk + 4 g + e (e < 4) or + 4 + e (e >= 4), which is this
    // lane's score 8 kk + e of the half.
    float psum = 0.f;
    bf16x8 pf[kTile / 16];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        // a masked score is -inf, and exp2(-inf) = 0 (muse is finite)
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[hf][i], c2, -muse));
        psum += p;
        pf[2 * hf + i / 8][i % 8] = (__bf16)p;
      }
    }
    l_run = l_run * alpha + psum;
    pv_step((j + kNV - 1) % kNV);  // tile j - 1 (or nothing before the first tile)
#pragma unroll
    for (int kk = 0; kk < kTile / 16; kk++) pf_prev[kk] = pf[kk];
    alpha_prev = alpha;
    pend = true;
    }
    // tile j + 1 has landed (tile j + 2 may still be in flight)
    if (ahead) wait_vm<kPerWave>();
    else wait_vm<0>();
    __syncthreads();
  }
  if (pend) {
    rescale_prev();
    pv_step((n_tiles - 1) % kNV);
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
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern::prefill_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kern::kLdsBytes);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.T + kern::kRowsWg - 1) / kern::kRowsWg) * (unsigned)a.H * (unsigned)a.B);
  hipLaunchKernelGGL(kern::prefill_kernel, grid, dim3(64 * kern::kWaves), kern::kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace mla
