// Sparse (DSA) decode over a bf16 latent cache, organised by head group.
//
// In DSA decode ("MLA & DSA 推理性能优化指南" §4.2; "MLA 最佳算子全景调研" §5)
// every query row of one (b, s) attends over the same list of selected
// tokens, and the list is short (topk), so there is too little work per
// (b, s) to give each compute unit a whole sequence.  The work item here is
// a head group: 32 query rows of one (b, s).  Its index list is cut into
// `hg_splits` contiguous ranges, one per workgroup, and each range into four
// quarters, one per wave.  Each wave is an independent decoder of the 32
// rows over its quarter: it gathers 16 tokens at a time into a private pair
// of LDS slots (direct HBM -> LDS copies of the selected rows), scores them
// with 16x16x32 MFMAs (S^T = K Q^T), runs the online softmax and
// accumulates O^T += V^T P^T with 32x32x16 MFMAs.  No barrier is shared
// between the waves until the end, where they merge their (max, sum, O)
// through LDS.  When a list has several ranges, each stores its normalised
// partial and a small second kernel merges them (a kernel boundary is the
// cheap way to make one compute unit's stores visible to another: an
// in-kernel release/acquire writes back the whole L2 of the XCD).  There is
// no scheduling pass.
// The head groups of one (b, s) and range are consecutive workgroups of one
// XCD: their gathers of the same rows meet in that XCD's L2.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace kern {

namespace {

// Region-A swizzle of a 16-row block of 1 KB latent rows: 16-byte chunk c
// of row r sits at position c ^ swz16(r).  swz16 is a linear bijection of
// r & 15; the 16x16 score-operand read (one chunk of 16 rows per 16 lanes)
// and the transposing value read (four chunks of 4 rows per 32 lanes) both
// cover every bank once with it.
__device__ __forceinline__ int swz16(int row) {
  return (((row & 3) << 2) | ((row >> 2) & 3)) ^ ((row & 4) >> 1);
}

// op over lanes l, l ^ 16, l ^ 32, l ^ 48: the four lanes that hold one query
// row's tokens in the 16x16 score layout.
__device__ __forceinline__ float quad_max(float x) {
  x = pair_max(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  x = pair_sum(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16x16x32 score MFMAs with the accumulator in ordinary registers (the
// accumulation registers all hold O).  Each of the two chains accumulates
// into exactly the same registers, which needs no wait states between
// MFMAs; mfma_settle() supplies the wait states before VALU reads.
__device__ __forceinline__ void mfma16_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_acc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_settle(f32x4& x, f32x4& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}

// copy16_s for a base address that lane reads (VALU) just wrote into the
// scalar registers: a vector memory instruction may read such registers only
// five wait states after the write, and the compiler does not count them
// for an assembly operand.
__device__ __forceinline__ void copy16_s_after_valu(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "{m0}"(lds));
}

// Source of the rows of invisible tokens: their weights are 0, and the
// values they contribute must be finite.
__device__ __attribute__((aligned(256))) const uint8_t kZeroRow[kBytesBf16Row] = {};

struct Hg {
  static constexpr int kTok = 16;                      // tokens per chunk
  static constexpr int kABlk = kTok * 1024;            // latent rows (V and score dims 0..511)
  static constexpr int kBBlk = kTok * 128;             // RoPE rows (score dims 512..575)
  static constexpr int kSlot = kABlk + kBBlk;          // 18 KB
  static constexpr int kWaveBytes = 2 * kSlot;         // two slots per wave
  static constexpr int kPOff = 4 * kWaveBytes;         // P (bf16 32 rows x 16 tokens) per wave
  static constexpr int kPBytes = 32 * 32;
  static constexpr int kStatOff = kPOff + 4 * kPBytes; // per wave and row: max, then sum
  static constexpr int kLookOff = kStatOff + 2 * 4 * 32 * 4;  // per wave: next round's indices, pages
  static constexpr int kLdsBytes = kLookOff + 4 * 1024;
  static constexpr int kRound = 128;                   // index entries looked up together
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(4 * 8 * 4096 <= kPOff, "merge buffers reuse the slots");
};

}  // namespace

__global__ __launch_bounds__(256, 1) void decode_bf16_sparse_hg(DecodeArgs a) {
  using Y = Hg;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lid = xcd_logical(blockIdx.x, gridDim.x);
  const int NR = a.hg_groups, S = a.hg_splits;
  const int hg = lid % NR;
  const int rest = lid / NR;
  const int split = rest % S;
  const int su = rest / S;
  const int item = su * NR + hg;
  const int b = su / a.Sq;
  const int L = max(ldc(a.seqlens + b), 0);
  const int rows = min(32, a.H - 32 * hg);
  const size_t row0 = (size_t)su * a.H + 32 * hg;  // flat query row of local row 0
  const int e_lo = min(a.topk, (split * 4 + w) * a.hg_span);
  const int e_hi = min(a.topk, e_lo + a.hg_span);
  const int nch = (e_hi - e_lo + Y::kTok - 1) / Y::kTok;
  const int32_t* idx_row = a.indices + (size_t)su * a.topk;
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;

  // This launch produces finished rows: a split merge pass run after it (the
  // staged interface) must leave them alone.
  if (split == 0 && hg == 0 && w == 0)
    for (int r = lane; r < a.row_blocks; r += 64) a.ws_meta[4 * (su * a.row_blocks + r) + 2] = 1;

  // ------------------------------------------------------------ lookups
  // A selected entry names a token of sequence b; it is visible when it is
  // below the sequence length and its page lies inside the block-table row
  // and the pool.  Token rows are page * 64 + (index & 63), or -1.
  // (loads from clamped, always valid addresses with the selects after
  // them: a load under a branch makes the compiler wait for it there)
  auto tok_of = [&](int i, int pg) __attribute__((always_inline)) -> int {
    const bool ok = i >= 0 && i < L && (i >> 6) < a.bt_stride && pg >= 0 && pg < a.num_pages;
    return ok ? pg * kPage + (i & 63) : -1;
  };

  uint8_t* const wbase = lds + w * Y::kWaveBytes;
  auto slot = [&](int c) __attribute__((always_inline)) -> uint8_t* { return wbase + (c & 1) * Y::kSlot; };
  uint8_t* const pb = lds + Y::kPOff + w * Y::kPBytes;

  // ------------------------------------------------------------ state
  bf16x8 qf[2][18];
  f32x16 o[16];
#pragma unroll
  for (int i = 0; i < 16; i++) o[i] = f32x16{};
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};

  // Chunk n of the wave (entries e_lo + 16 n ..) in terms of the current
  // round's token rows t0 (entries + lane) and t1 (entries + 64 + lane).
  int t0 = -1, t1 = -1;
  struct Next {
    int lst, lo;        // token-row register and first lane of the chunk
    unsigned vm;        // visible tokens of the chunk (bit j: token j)
    int rope0, rope1;   // per lane: token row of RoPE copy 0 / 1
    uint32_t sa;        // LDS address of the chunk's slot
    uint32_t alo, ahi;  // per lane: address of the latent row of lst (the zero row if invisible)
  };
  // (the token rows come in by value: a select between two variables in
  // memory would keep them there)
  auto setup = [&](int n, int ta, int tb) __attribute__((always_inline)) -> Next {
    Next d;
    const int j = n & 7;
    d.lst = j < 4 ? ta : tb;
    d.lo = 16 * (j & 3);
    d.vm = (unsigned)(__builtin_amdgcn_ballot_w64(d.lst >= 0) >> d.lo) & 0xffffu;
    d.rope0 = __shfl(d.lst, d.lo + (lane >> 3));
    d.rope1 = __shfl(d.lst, d.lo + 8 + (lane >> 3));
    d.sa = lds_addr(slot(n));
    // the 16 copy sources of the chunk, computed by all lanes at once: a copy
    // then only reads its row's address out of lane lo + k
    const uint64_t ra = d.lst >= 0 ? reinterpret_cast<uint64_t>(a.kv) + (uint64_t)(uint32_t)d.lst * kBytesBf16Row
                                   : reinterpret_cast<uint64_t>(kZeroRow);
    d.alo = (uint32_t)ra;
    d.ahi = (uint32_t)(ra >> 32);
    return d;
  };
  // Copy k of a chunk: k < 16 the latent row of token k (lane = 16-byte
  // position), k = 16, 17 the RoPE rows of tokens 8 (k - 16) .. +7 (lane /
  // 8 = row, lane % 8 = position).  Invisible tokens copy the zero row, so
  // every chunk issues the same copies and the loop has no branches.
  auto copy = [&](int k, Next d) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // per-lane offsets are not kept live through the loop
    if (k < Y::kTok) {
      // the row address is wave-uniform: two lane reads into scalar registers
      const uint32_t lo32 = __builtin_amdgcn_readlane(d.alo, d.lo + k);
      const uint32_t hi32 = __builtin_amdgcn_readlane(d.ahi, d.lo + k);
      const uint64_t su64 = ((uint64_t)hi32 << 32) | lo32;
      copy16_s_after_valu(reinterpret_cast<const void*>(su64), (uint32_t)((ln ^ swz16(k)) << 4), d.sa + k * 1024);
    } else {
      const int jb = k - Y::kTok;
      const int row = 8 * jb + (ln >> 3);
      const int t = jb ? d.rope1 : d.rope0;
      const uint8_t* rowp = t >= 0 ? a.kv + (size_t)t * kBytesBf16Row + 1024 : kZeroRow;
      copy16_v(rowp + (((ln & 7) ^ ((row >> 1) & 7)) << 4), d.sa + Y::kABlk + jb * 1024);
    }
  };

  // The group's 32 query rows, once per workgroup, issued first so that their
  // round trip overlaps the index and page lookups': 36 direct copies of whole
  // rows (9 per wave) into slot 1 of waves 0 (rows 0..15) and 1 (rows
  // 16..31), in the layout of a chunk, so that every wave reads its score
  // operand out of LDS as it reads the cache rows.  Rows past the head count
  // take row 0's query; they are never written out.
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 9; i++) {
      const int q = 9 * w + i;  // wave-uniform
      if (q < 32) {
        const int rb = q >> 4, k = q & 15;
        const size_t grow = row0 + (q < rows ? q : 0);
        copy16_s(a.q_nope + grow * kDC, (uint32_t)((ln ^ swz16(k)) << 4),
                 lds_addr(lds + rb * Y::kWaveBytes + Y::kSlot + k * 1024));
      } else {
        const int jb = q - 32, rb = jb >> 1, row = 8 * (jb & 1) + (ln >> 3);
        const int r = 16 * rb + row;
        const size_t grow = row0 + (r < rows ? r : 0);
        copy16_v(reinterpret_cast<const uint8_t*>(a.q_rope + grow * kDR) + (((ln & 7) ^ ((row >> 1) & 7)) << 4),
                 lds_addr(lds + rb * Y::kWaveBytes + Y::kSlot + Y::kABlk + (jb & 1) * 1024));
      }
    }
  }
  asm volatile("" ::: "memory");
  // Round 0 lookups.  The block-table row is fetched towards L2 beside the
  // index loads (into a scratch area of LDS), so the dependent page lookups
  // find it there.  Issue order: index entries, then their pages (vector
  // loads retire in order); the empty asm statements with a memory clobber
  // keep the compiler from reordering the groups.
  const int ea = e_lo + lane, eb = ea + 64;
  int va = -1, vb = -1, pa = -1, pbg = -1;
  if (nch > 0) {
    const int nb = min(a.bt_stride, 1024);  // entries: up to 4 KB per row
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int e = 256 * k + 64 * w + lane;
      if (e < nb) copy4_v(bt_row + e, lds_addr(lds + Y::kLookOff + w * 1024 + k * 256));
    }
    va = idx_row[min(ea, e_hi - 1)];
    vb = idx_row[min(eb, e_hi - 1)];
    asm volatile("" ::: "memory");
    pa = bt_row[min(max(va >> 6, 0), a.bt_stride - 1)];
    pbg = bt_row[min(max(vb >> 6, 0), a.bt_stride - 1)];
    asm volatile("" ::: "memory");
  }
  if (nch > 0) {
    const int i0 = ea < e_hi ? va : -1, i1 = eb < e_hi ? vb : -1;
    t0 = tok_of(i0, pa);
    t1 = tok_of(i1, pbg);
    const Next d0 = setup(0, t0, t1);
    wait_lds();
#pragma unroll
    for (int k = 0; k < Y::kTok + 2; k++) copy(k, d0);
    wait_vm<Y::kTok + 2>();  // this wave's query copies (issued before chunk 0's) have landed
  } else {
    wait_vm<0>();
  }
  __syncthreads();  // every wave's query copies are in LDS
  if (nch > 0) {
    const int r16 = lane & 15, g4 = lane >> 4, y = swz16(r16);
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      const uint8_t* qs = lds + rb * Y::kWaveBytes + Y::kSlot;
#pragma unroll
      for (int ks = 0; ks < 16; ks++)
        qf[rb][ks] = *reinterpret_cast<const bf16x8*>(qs + r16 * 1024 + 256 * (ks >> 2) +
                                                       64 * ((ks & 3) ^ (y >> 2)) + 16 * ((g4 ^ y) & 3));
#pragma unroll
      for (int k = 0; k < 2; k++)
        qf[rb][16 + k] = *reinterpret_cast<const bf16x8*>(qs + Y::kABlk + r16 * 128 +
                                                          (((4 * k + g4) ^ ((r16 >> 1) & 7)) << 4));
    }
    // take delivery here: a wait left to the compiler would land in the loop
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
      for (int ks = 0; ks < 18; ks++) asm volatile("" : "+v"(qf[rb][ks]));
  }
  __syncthreads();  // slot 1 of waves 0 and 1 is free for chunk 1

  // ------------------------------------------------------------ main loop
  unsigned vm_cur = 0;
  if (nch > 0) vm_cur = (unsigned)(__builtin_amdgcn_ballot_w64(t0 >= 0)) & 0xffffu;
  // Next round's lookups land in LDS through direct copies, which the
  // chunk waits cover: indices at look[0..127], then their pages at
  // look[128..255] (-1 where there is nothing to look up).
  int* const look = reinterpret_cast<int*>(lds + Y::kLookOff + w * 1024);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int y = swz16(r16);
#pragma unroll 1
  for (int c = 0; c < nch; c++) {
    wait_vm<0>();  // chunk c (and every older load) has landed
    const int j = c & 7;
    const bool next_round = 8 * ((c >> 3) + 1) < nch;
    if (next_round) {
      const int e_next = e_lo + Y::kRound * ((c >> 3) + 1);
      if (j == 1) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int e = e_next + 64 * h + lane;
          if (e < e_hi) copy4_v(idx_row + e, lds_addr(look + 64 * h));
          else look[64 * h + lane] = -1;
        }
      }
      if (j == 4) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int i = look[64 * h + lane];
          if (i >= 0 && i < L && (i >> 6) < a.bt_stride) copy4_v(bt_row + (i >> 6), lds_addr(look + 128 + 64 * h));
          else look[128 + 64 * h + lane] = -1;
        }
      }
      if (j == 7) {
        t0 = tok_of(look[lane], look[128 + lane]);
        t1 = tok_of(look[64 + lane], look[192 + lane]);
      }
    }
    // chunk c + 1 (past the end: an all-invisible chunk, whose copies of
    // the zero row land in a slot nothing reads again)
    if (c + 1 >= nch) {
      t0 = -1;
      t1 = -1;
    }
    const Next nd = setup(c + 1, t0, t1);
    wait_lds();

    // ---- S^T[token][row] over 576 dims: k-step ks reads 16-byte chunk
    // 4 ks + (lane >> 4) of token (lane & 15); ks < 16 from region A, 16 and
    // 17 from region B.  Chunk c + 1's copies are spread over the k-steps.
    const uint32_t sa = lds_addr(slot(c)), sb = sa + Y::kABlk;
    uint32_t offA[4], offB[2];
#pragma unroll
    for (int kl = 0; kl < 4; kl++)
      offA[kl] = sa + r16 * 1024 + 64 * (kl ^ (y >> 2)) + 16 * ((g4 ^ y) & 3);
#pragma unroll
    for (int k = 0; k < 2; k++) offB[k] = sb + r16 * 128 + (((4 * k + g4) ^ ((r16 >> 1) & 7)) << 4);
    constexpr int kLead = 4, kRingK = kLead + 2;
    bf16x8 ring[kRingK];
    auto rd = [&](auto KS) __attribute__((always_inline)) {
      constexpr int ks = decltype(KS)::value;
      if constexpr (ks < 16) lds_rd16<256 * (ks >> 2)>(ring[ks % kRingK], offA[ks & 3]);
      else lds_rd16<0>(ring[ks % kRingK], offB[ks - 16]);
    };
    f32x4 s0, s1;
    unroll<kLead>(rd);
    unroll<18>([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      lds_ready<(kLead - 1 < 17 - ks ? kLead - 1 : 17 - ks)>(ring[ks % kRingK]);
      copy(ks, nd);
      if constexpr (ks == 0) {
        mfma16_first(s0, ring[0], qf[0][0]);
        mfma16_first(s1, ring[0], qf[1][0]);
      } else {
        mfma16_acc(s0, ring[ks % kRingK], qf[0][ks]);
        mfma16_acc(s1, ring[ks % kRingK], qf[1][ks]);
      }
      if constexpr (ks + kLead < 18) rd(std::integral_constant<int, ks + kLead>{});
    });
    mfma16_settle(s0, s1);

    // ---- online softmax: lane holds rows 16 rb + (lane & 15), tokens
    // 4 (lane >> 4) + i.  P goes to LDS in the order the P.V operand reads
    // it: row r, 16-byte chunk h at position h ^ ((r >> 3) & 1) holds tokens
    // 4h + {0..3, 8..11}.
    const float c2 = a.scale_log2;
    const unsigned vmk = vm_cur >> (4 * g4);
    float mt[2];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const bool ok = (vmk >> i) & 1u;
      s0[i] = ok ? s0[i] : kNegInf;
      s1[i] = ok ? s1[i] : kNegInf;
    }
    mt[0] = quad_max(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3]))) * c2;
    mt[1] = quad_max(fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))) * c2;
    const float mn0 = fmaxf(m_run[0], mt[0]), mn1 = fmaxf(m_run[1], mt[1]);
    const bool need = mn0 > m_run[0] + kRescaleSlack || mn1 > m_run[1] + kRescaleSlack;
    const bool moved = __builtin_amdgcn_ballot_w64(need) != 0;
    const float al0 = (moved && m_run[0] != kNegInf) ? __builtin_amdgcn_exp2f(m_run[0] - mn0) : 1.f;
    const float al1 = (moved && m_run[1] != kNegInf) ? __builtin_amdgcn_exp2f(m_run[1] - mn1) : 1.f;
    m_run[0] = moved ? mn0 : m_run[0];
    m_run[1] = moved ? mn1 : m_run[1];
    const float mu0 = m_run[0] == kNegInf ? 0.f : m_run[0];
    const float mu1 = m_run[1] == kNegInf ? 0.f : m_run[1];
    float ps0 = 0.f, ps1 = 0.f;
    bf16x2 pw0[2], pw1[2];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c2, -mu0));
      const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c2, -mu1));
      ps0 += p;
      ps1 += q;
      pw0[i >> 1][i & 1] = (__bf16)p;
      pw1[i >> 1][i & 1] = (__bf16)q;
    }
    l_run[0] = l_run[0] * al0 + ps0;
    l_run[1] = l_run[1] * al1 + ps1;
    {
      const int pos = 8 * (g4 >> 1);
      const int ra = r16, rb = 16 + r16;
      *reinterpret_cast<u32x2*>(pb + ra * 32 + (((g4 & 1) ^ ((ra >> 3) & 1)) << 4) + pos) =
          u32x2{__builtin_bit_cast(unsigned, pw0[0]), __builtin_bit_cast(unsigned, pw0[1])};
      *reinterpret_cast<u32x2*>(pb + rb * 32 + (((g4 & 1) ^ ((rb >> 3) & 1)) << 4) + pos) =
          u32x2{__builtin_bit_cast(unsigned, pw1[0]), __builtin_bit_cast(unsigned, pw1[1])};
    }
    // O^T rows: lane holds row lane & 31 = 16 ((lane >> 4) & 1) + (lane & 15)
    const float al = ((lane >> 4) & 1) ? al1 : al0;
    if (__builtin_amdgcn_ballot_w64(al != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < 16; db++) acc_scale(o[db], al);
    }

    // ---- O^T[dim][row] += V^T[dim][token] P^T[token][row], 32 dims per MFMA
    {
      int lnv = lane;
      asm volatile("" : "+v"(lnv));
      const int G16v = lnv >> 4, i16v = lnv & 15;
      const int row0v = 4 * (G16v >> 1) + (i16v >> 2);  // token of the first read; the second is 8 further
      const int wv = 2 * (G16v & 1) + ((i16v >> 1) & 1);
      const int vy0 = wv ^ swz16(row0v), vy1 = wv ^ swz16(row0v + 8);
      const uint8_t* cur = slot(c) + row0v * 1024 + 8 * (i16v & 1);
      const int pr = lnv & 31;
      const bf16x8 pbv =
          *reinterpret_cast<const bf16x8*>(pb + pr * 32 + (((lnv >> 5) ^ ((pr >> 3) & 1)) << 4));
#pragma unroll
      for (int i = 0; i < 16; i++) {
        // four dim blocks' value reads in flight at a time
        if (i % 4 == 0 && i > 0) __builtin_amdgcn_sched_barrier(0);
        // slot i holds dim block (i + 4 w) & 15: the low two bits are i's
        const int hi = 256 * (((i >> 2) + w) & 3);
        const uint8_t* p0 = cur + hi + (((4 * (i & 3)) ^ vy0) << 4);
        const uint8_t* p1 = cur + 8 * 1024 + hi + (((4 * (i & 3)) ^ vy1) << 4);
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p0));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p1));
        const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pbv, o[i], 0, 0, 0);
      }
    }
    wait_lds();  // this chunk's slot and P are read before they are refilled
    vm_cur = nd.vm;
  }
  wait_vm<0>();

  // ------------------------------------------------------------ merge
  // Accumulator slot i of wave w holds dims 32 ((i + 4 w) & 15) .. +31, so
  // slots 0..3 are dims 128 w .. +127, the quarter wave w owns.  (1) The four
  // waves' running maxima and sums per row give each wave its weight; (2) in
  // three passes k = 1..3 every wave hands slots 4k..4k+3 (dims of wave
  // (w + k) & 3) to their owner through LDS, which adds them to its own.
  const float lt0 = quad_sum(l_run[0]), lt1 = quad_sum(l_run[1]);
  float* const stm = reinterpret_cast<float*>(lds + Y::kStatOff);
  __syncthreads();  // every wave is done with its slots
  if (lane < 16) {
    stm[32 * w + lane] = m_run[0];
    stm[32 * w + 16 + lane] = m_run[1];
    stm[128 + 32 * w + lane] = lt0;
    stm[128 + 32 * w + 16 + lane] = lt1;
  }
  __syncthreads();
  const int r = lane & 31;
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < 4; k++) M = fmaxf(M, stm[32 * k + r]);
  float Lsum = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int k = 0; k < 4; k++) Lsum += stm[128 + 32 * k + r] * __builtin_amdgcn_exp2f(stm[32 * k + r] - M);
  }
  const bool has = Lsum > 0.f;
  const float mown = stm[32 * w + r];
  const float f = (has && mown != kNegInf) ? __builtin_amdgcn_exp2f(mown - M) / Lsum : 0.f;
  const float lse2 = has ? M + __log2f(Lsum) : kNegInf;
  // The owned quarter moves to ordinary registers (the query registers are
  // free now), weighted; the other three quarters are weighted as they are
  // handed over.
  float own[64];
#pragma unroll
  for (int jj = 0; jj < 4; jj++)
#pragma unroll
    for (int e = 0; e < 16; e++) own[16 * jj + e] = acc_get(o[jj], e) * f;

  // slots SB..SB+3 to `buf` (4 KB per slot, 1 KB of consecutive bytes per
  // store) times sc
  auto put4 = [&](auto SB, float* buf, float sc) __attribute__((always_inline)) {
    constexpr int sb = decltype(SB)::value;
#pragma unroll
    for (int jj = 0; jj < 4; jj++)
#pragma unroll
      for (int q = 0; q < 4; q++)
        *reinterpret_cast<f32x4*>(buf + (jj * 4 + q) * 256 + lane * 4) =
            f32x4{acc_get(o[sb + jj], 4 * q), acc_get(o[sb + jj], 4 * q + 1), acc_get(o[sb + jj], 4 * q + 2),
                  acc_get(o[sb + jj], 4 * q + 3)} * sc;
  };
  float* const X = reinterpret_cast<float*>(lds);  // two regions of 4 x 16 KB
  unroll<3>([&](auto K) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value + 1;
    float* const reg = X + ((k & 1) ? 0 : 16384);
    put4(std::integral_constant<int, 4 * k>{}, reg + 4096 * ((w + k) & 3), f);
    __syncthreads();
    const float* buf = reg + 4096 * w;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(buf + i * 256 + lane * 4);
#pragma unroll
      for (int e = 0; e < 4; e++) own[4 * i + e] += v[e];
    }
  });

  // ------------------------------------------------------------ results
  const bool row_ok = r < rows;
  // this wave's dims times `inv` as bf16, and the rows' lse
  auto emit = [&](float inv, float lse_nat) __attribute__((always_inline)) {
    if (!row_ok) return;
    uint16_t* dst = a.out + (row0 + r) * kDC + 128 * w + 4 * (lane >> 5);
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float* x = own + 16 * jj + 4 * q;
        bf16x2 p0 = {(__bf16)(x[0] * inv), (__bf16)(x[1] * inv)};
        bf16x2 p1 = {(__bf16)(x[2] * inv), (__bf16)(x[3] * inv)};
        *reinterpret_cast<u32x2*>(dst + 32 * jj + 8 * q) =
            u32x2{__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1)};
      }
    }
    if (w == 0 && lane < 32) a.lse[row0 + r] = lse_nat;
  };
  if (S == 1) {
    emit(1.f, has ? lse2 * kLn2 : kNegInf);
    return;
  }

  // Several ranges: store this range's normalised partial (each wave its
  // quarter, in fragment order) as fp16 divided by the row's largest
  // magnitude in the quarter (so every value lies in [-1, 1]), that scale,
  // and the range's log2-sum-exp; combine_hg merges them.
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 64; i++) mx = fmaxf(mx, fabsf(own[i]));
  mx = pair_max(mx);  // lanes r and r + 32 hold the row's other dims
  const float sc = mx > 0.f ? mx : 1.f;
  const float inv = 1.0f / sc;
  const size_t part = (size_t)item * S + split;
  _Float16* const pdst = reinterpret_cast<_Float16*>(a.ws_po) + part * (16 * 1024) + w * 4096;
#pragma unroll
  for (int i = 0; i < 16; i++)
    *reinterpret_cast<f16x4*>(pdst + i * 256 + lane * 4) =
        f16x4{(_Float16)(own[4 * i] * inv), (_Float16)(own[4 * i + 1] * inv), (_Float16)(own[4 * i + 2] * inv),
              (_Float16)(own[4 * i + 3] * inv)};
  if (lane < 32) a.ws_psc[part * 128 + w * 32 + r] = sc;
  if (w == 0 && lane < 32) a.ws_plse[part * 32 + r] = lse2;
}

// Merge of the ranges of every item, in range order.  A partial holds 4096
// pieces of four values in fragment order (piece t: t >> 10 = the wave that
// stored it, lane t & 63), i.e. row t & 31 and dims
// 32 (t >> 8) + 8 ((t >> 6) & 3) + 4 ((t >> 5) & 1) .. +3.  Thread u of the
// item's 2048 takes pieces 2u and 2u + 1, 16 contiguous bytes: rows r0 and
// r0 + 1 at the same four dims.
__global__ __launch_bounds__(256) void combine_hg(DecodeArgs a) {
  const int item = blockIdx.x;
  const int t0 = 2 * (blockIdx.y * 256 + threadIdx.x);
  const int NR = a.hg_groups, S = a.hg_splits;
  const int hg = item % NR, su = item / NR;
  const int rows = min(32, a.H - 32 * hg);
  const int r0 = t0 & 31;
  if (r0 >= rows) return;
  const bool second = r0 + 1 < rows;
  const size_t row0 = (size_t)su * a.H + 32 * hg + r0;
  const int d = 32 * (t0 >> 8) + 8 * ((t0 >> 6) & 3) + 4 * ((t0 >> 5) & 1);
  const int qw = t0 >> 10;  // the quarter of the dims (the wave that stored it)
  const size_t base = (size_t)item * S;
  const _Float16* const po = reinterpret_cast<const _Float16*>(a.ws_po) + 4 * t0;
  float mx0 = kNegInf, mx1 = kNegInf;
  for (int s = 0; s < S; s++) {
    const float2 l = *reinterpret_cast<const float2*>(a.ws_plse + (base + s) * 32 + r0);
    mx0 = fmaxf(mx0, l.x);
    mx1 = fmaxf(mx1, l.y);
  }
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float ws0 = 0.f, ws1 = 0.f;
  for (int s = 0; s < S; s++) {
    const float2 l = *reinterpret_cast<const float2*>(a.ws_plse + (base + s) * 32 + r0);
    const float2 sc = *reinterpret_cast<const float2*>(a.ws_psc + (base + s) * 128 + qw * 32 + r0);
    const f16x8 h = *reinterpret_cast<const f16x8*>(po + (base + s) * (16 * 1024));
    // weight 0 for an empty range (lse -inf) and for a row with no token
    const float w0 = mx0 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(l.x - mx0);
    const float w1 = mx1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(l.y - mx1);
    ws0 += w0;
    ws1 += w1;
    const float f0 = w0 * sc.x, f1 = w1 * sc.y;
    acc0 += f0 * f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    acc1 += f1 * f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
  }
  const bool lse_writer = t0 < 32;
  auto put = [&](size_t row, const f32x4& acc, float wsum, float mx) {
    uint16_t* dst = a.out + row * kDC + d;
    if (mx == kNegInf) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{0u, 0u};
      if (lse_writer) a.lse[row] = kNegInf;
      return;
    }
    const float inv = 1.0f / wsum;
    const bf16x2 p0 = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
    const bf16x2 p1 = {(__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)};
    *reinterpret_cast<u32x2*>(dst) = u32x2{__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1)};
    if (lse_writer) a.lse[row] = (mx + __log2f(wsum)) * kLn2;
  };
  put(row0, acc0, ws0, mx0);
  if (second) put(row0 + 1, acc1, ws1, mx1);
}

}  // namespace kern

hipError_t launch_sparse_hg(const Geometry& g, const DecodeArgs& a, hipStream_t stream) {
  using kern::decode_bf16_sparse_hg;
  using kern::Hg;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_bf16_sparse_hg),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Hg::kLdsBytes);
  if (e != hipSuccess) return e;
  const long long grid = (long long)g.n_su * g.hg_splits * g.hg_groups;
  hipLaunchKernelGGL(decode_bf16_sparse_hg, dim3((unsigned)grid), dim3(256), Hg::kLdsBytes, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || g.hg_splits == 1) return e;
  hipLaunchKernelGGL(kern::combine_hg, dim3((unsigned)(g.n_su * g.hg_groups), 8), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
