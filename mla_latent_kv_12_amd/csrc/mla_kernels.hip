// HIP kernels of the weight-absorbed MLA decode path, written for gfx950 (CDNA4).
//
// The method ("MLA 在极长上下文下的显存带宽突围", section "运行期矩阵吸收避免潜在
// 张量展开"): with W_UK absorbed into the query, every head scores the cached
// 576-dim latent row directly, Score = q~ c^T + q^R k^R^T, and ("MLA & DSA 推理性
// 能优化指南" §1.1) the same latent c is the value.  Decode is bound by reading
// the cache (§4 of that guide), so the kernel is organised around reading each
// 64-token page once from HBM and reusing it from LDS for every query row of
// its sequence:
//
//   plan_kernel     split-KV partition of all 64-token tiles over the
//                   persistent workgroups, with a fixed cost per split
//   decode_*_r{4,2,1w}
//                   per workgroup: stream its 32-token chunks HBM -> LDS
//                   (direct global->LDS loads into a ring of slots,
//                   XOR-swizzled rows), S^T = K Q^T and O^T += V^T P^T on
//                   bf16 MFMA 32x32x16 with fp32 accumulation, online softmax
//                   in the log2 domain; fp8 e4m3 chunks are converted to bf16
//                   in registers (exact)
// (the log-sum-exp merge of split units' partial results is in mla_combine.hip)
//
// Wave roles: the R waves of a workgroup (R = 4, 2, 1 for units of up to
// 128, 64, 32 query rows) share each chunk in LDS.  For the scores a wave
// owns 32 query rows; for P.V it owns 512/R output dims of all the unit's
// rows.  One-wave workgroups run four (fp8) or two (bf16) to a compute unit.
#include "mla_device.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {
namespace kern {

template <bool SPARSE>
__global__ __launch_bounds__(256) void plan_kernel(DecodeArgs a) {
  plan_work<SPARSE>(a);
}

// Copy source for cache rows that are not visible: zeros (their weights are
// 0, and the values they contribute must be finite).
__device__ __attribute__((aligned(256))) const uint8_t kZeroSrc[1280] = {};

// bf16 region-A swizzle of a cached row: the 16-byte chunk c of row r sits at
// position c ^ sw16(r).  The score operand reads one chunk of 16 consecutive
// rows per 16 lanes (sw16 is a bijection on r & 15) and the transposed value
// reads take 4 chunks of 4 consecutive rows per 32 lanes; both cover every
// bank once.
__device__ __forceinline__ int sw16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// ---------------------------------------------------------------------------
// Main kernel for units of 33..128 query rows ("wide" units).
//
// The R waves of a workgroup work on the same 32-token chunk of the cache
// (half a page).  For the scores each wave owns 32 query rows (its Q stays
// in registers); for P.V each wave owns 512/R output dims of all rows, with
// P passed between the waves through LDS, so each chunk's values are read
// out of LDS (transposed) once.
//
// Pipeline.  The workgroup walks its chunks ("items") in order, over all
// the units its share of the work touches.  At step s it computes item s,
// copies item s+3 from HBM into LDS (those copies are spread between the
// score MFMAs of item s), and looks up what item s+6 needs: its page
// (dense), or its 32 page numbers (sparse; the 32 token positions of item
// s+9 are fetched at the same time).  Every lookup lands in LDS through the
// same direct copies, so nothing in the loop waits on a scalar load and
// three chunks (108 KB bf16) are in flight per compute unit.
//
// Item descriptors (LDS ring, 8 ints): unit (-1 past the end of the
// workgroup's work), 2*tile + half (-1: no chunk), page (dense) or sequence
// (sparse), sequence length, mask of visible tokens (sparse).
// ---------------------------------------------------------------------------
template <bool FP8, bool SPARSE, int R>
struct Wide {
  static constexpr int kThreads = 64 * R;
  static constexpr int kEB = FP8 ? 1 : 2;
  static constexpr int kRowBytes = kD * kEB;        // 1152 | 576 per cached token
  static constexpr int kABytes = kDC * kEB;         // 1024 | 512: latent part of a row
  static constexpr int kRows = 32;                  // tokens per chunk
  // Multi-wave workgroups pipeline each chunk's P.V into the next chunk's
  // step, where it overlaps the softmax (one barrier per chunk).
  static constexpr bool kPipe = R == 4 && !FP8;
  // A chunk occupies one block of the region-A ring (latent part, also the
  // P.V operand) and one block of the region-B ring (RoPE part, fp8 scales),
  // which is free as soon as the scores are done.
  static constexpr int kABlk = kRows * kABytes;
  static constexpr int kScaleOffB = kRows * kDR * kEB;  // fp8 scales in a region-B block
  static constexpr int kBBlk = kScaleOffB + (FP8 ? 128 : 0);
  // One-wave workgroups (units of <= 32 rows) run four to a compute unit
  // (fp8; bf16 slots fit two) and keep two chunks in LDS.
  static constexpr int kSlots = (R == 1) ? 2 : 4;
  static constexpr int kSlotsB = kPipe ? kSlots - 1 : kSlots;
  static constexpr int kNA = FP8 ? 16 : 32;         // 1 KB copies of region A
  static constexpr int kNB = FP8 ? 2 : 4;           // 1 KB copies of region B
  static constexpr int kNCopy = kNA + kNB + (FP8 ? 1 : 0);  // (+ the 32 scales)
  // every wave issues the same number of copies per item (padded with
  // 4-byte dummy copies), so one wait count serves all of them
  static constexpr int kPerWave = (kNCopy + R - 1) / R;
  static_assert(kNA % R == 0, "region-A copies must split evenly over the waves");
  static constexpr int kLook = SPARSE ? 2 : 0;      // lookup copies per step (wave 0)
  // Copies of item z are issued while item z - kLeadDma is computed: the
  // pipelined step also still reads item z - kLeadDma - 1 (its P.V).
  static constexpr int kLeadDma = kPipe ? kSlots - 2 : kSlots - 1;
  static constexpr int kLeadPage = 2 * kLeadDma;
  static constexpr int kLeadCur = SPARSE ? 3 * kLeadDma : kLeadPage;
  static constexpr int kRing = kLeadCur < 8 ? 8 : 16;
  static_assert(kRing > kLeadCur, "descriptor ring too short");
  static constexpr int kBOff = kSlots * kABlk;
  static constexpr int kDescOff = kBOff + kSlotsB * kBBlk;
  static constexpr int kIdxOff = kDescOff + (SPARSE ? kRing * 32 : 0);
  static constexpr int kPgOff = kIdxOff + (SPARSE ? kRing * 128 : 0);
  static constexpr int kPOff = kPgOff + (SPARSE ? kRing * 128 : 0);
  // P and the rescale factors are double-buffered when pipelined (chunk s
  // writes them while chunk s-1's are read); the end-of-segment merge
  // buffers then reuse the rescale buffers.
  static constexpr int kNPBuf = kPipe ? 2 : 1;
  static constexpr int kPBytes = 32 * R * 64;
  static constexpr int kAlphaOff = kPOff + kNPBuf * kPBytes;
  static constexpr int kMrgOff = kPipe ? kAlphaOff : kAlphaOff + 32 * R * 4;
  static constexpr int kDummyOff = kMrgOff + 2 * 32 * R * 4;
  static constexpr int kLdsBytes = kDummyOff + 64;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(4 * 2 * (kFoldUnits + 1) <= kSlots * kABlk,
                "the self-schedule's scratch fits in the chunk ring");
  static_assert(kABlk % 1024 == 0 && kBBlk % 16 == 0 && kBOff % 16 == 0, "block alignment");
  // vector-memory operations wave w issues per step: its copies, plus the
  // lookups of wave 0
  static constexpr int per_step(int w) { return kPerWave + (w == 0 ? kLook : 0); }
};

template <bool FP8, bool SPARSE, int R>
__device__ __forceinline__ void decode_wide(const DecodeArgs& a) {
  using W = Wide<FP8, SPARSE, R>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int rg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int wg = xcd_logical(blockIdx.x, gridDim.x);

  // Item z's blocks in the two rings, its P buffer and rescale factors.
  // (item numbers are never negative: unsigned remainders are cheaper)
  auto blk_a = [&](int z) -> uint8_t* { return lds + ((unsigned)z % W::kSlots) * W::kABlk; };
  auto blk_b = [&](int z) -> uint8_t* { return lds + W::kBOff + ((unsigned)z % W::kSlotsB) * W::kBBlk; };
  auto pbuf_of = [&](int z) -> uint8_t* { return lds + W::kPOff + (W::kPipe ? (z & 1) * W::kPBytes : 0); };
  auto alpha_of = [&](int z) -> float* {
    return reinterpret_cast<float*>(lds + W::kAlphaOff + (W::kPipe ? (z & 1) * 32 * R * 4 : 0));
  };
  int* const desc_ring = reinterpret_cast<int*>(lds + W::kDescOff);
  int* const idx_ring = reinterpret_cast<int*>(lds + W::kIdxOff);
  int* const pg_ring = reinterpret_cast<int*>(lds + W::kPgOff);
  float* const mrg = reinterpret_cast<float*>(lds + W::kMrgOff);
  int* const dummy = reinterpret_cast<int*>(lds + W::kDummyOff);
  auto desc = [&](int x) -> int* { return desc_ring + (x & (W::kRing - 1)) * 8; };
  struct Desc {
    int u, th, p2, L;  // unit, 2*tile+half, page | sequence, length
  };
  auto read_desc = [&](int x) -> Desc {
    const i32x4 v = *reinterpret_cast<const i32x4*>(desc(x));
    return Desc{__builtin_amdgcn_readfirstlane(v[0]), __builtin_amdgcn_readfirstlane(v[1]),
                __builtin_amdgcn_readfirstlane(v[2]), __builtin_amdgcn_readfirstlane(v[3])};
  };

  // ------------------------------------------------------------ cursor
  // The lookup cursor walks the workgroup's chunks: unit cu (-1 once done),
  // chunk cc (tile cc / 2, half cc % 2), chunk range end chi, sequence
  // (dense b / sparse su) cs and its length cL.  Every wave runs it (uniform
  // scalar code).
  // This workgroup's share of the schedule: computed here (the LDS ring is
  // still free) unless a scheduling launch already wrote it.
  WgSched sc;
  if (a.fold_plan) {
    sc = sched_in_wg<SPARSE>(a, reinterpret_cast<int*>(lds), tid, wg);
  } else {
    sc.u0 = ldc(a.ws_work + 2 * wg);
    sc.t0 = ldc(a.ws_work + 2 * wg + 1);
    sc.u1 = ldc(a.ws_work + 2 * wg + 2);
    sc.t1 = ldc(a.ws_work + 2 * wg + 3);
    sc.q = max((ldc(a.ws_cost + a.n_units) + a.num_wg - 1) / a.num_wg, kMinWgCost);
    const int uc = min(sc.u0, a.n_units - 1);
    sc.c0 = ldc(a.ws_cost + uc);
    sc.b0 = ldc(a.ws_meta + 4 * uc + 1);
  }
  const int u_end = sc.u1, t_end = sc.t1;
  int cu = sc.u0, cc = sc.t0, chi = 0, cs = 0, cL = 0;
  auto enter = [&]() {  // settle (cu, cc) on the next unit with a chunk left
    for (;;) {
      if (cu > u_end || cu >= a.n_units) {
        cu = -1;
        return;
      }
      chi = (cu == u_end) ? t_end : unit_chunks(a, SPARSE, cu);
      if (cc < chi) break;
      cu++;
      cc = 0;
    }
    cs = cu / a.row_blocks;
    const int b = SPARSE ? cs / a.Sq : cs;
    cL = max(ldc(a.seqlens + b), 0);
  };
  auto next = [&]() {
    if (cu < 0) return;
    cc++;
    if (cc >= chi) {
      cu++;
      cc = 0;
      enter();
    }
  };
  enter();
  if (cu < 0) return;  // uniform: this workgroup has no work

  // Dense chunks are described in scalar registers, compactly: unit, page
  // (read from the block table by a scalar load, checked at use) and
  // 2 * (tokens left from the chunk's first token) + half-page.
  struct DD {
    int u, pg, remh;
  };
  auto cursor_desc = [&]() -> DD {
    DD d;
    d.u = cu;
    const int ct = cc >> 1;
    d.remh = 2 * (cL - 32 * cc) + (cc & 1);
    d.pg = (cu >= 0 && ct < a.bt_stride) ? ldc(a.block_table + (size_t)cs * a.bt_stride + ct) : -1;
    return d;
  };
  // Visible rows at the start of a dense chunk (0 when it has no page).
  auto dd_nvalid = [&](const DD& d) -> int {
    const bool ok = d.u >= 0 && d.pg >= 0 && d.pg < a.num_pages;
    return ok ? min(max(d.remh >> 1, 0), 32) : 0;
  };

  // Sparse: writes the descriptor of the cursor's item x and starts the
  // lookups of its 32 token positions (wave 0); always exactly one copy, so
  // the counts stay exact.
  auto lookup = [&](int x) {
    if (rg != 0) return;
    int* d = desc(x);
    const int th = cu >= 0 ? cc : -1;
    if constexpr (SPARSE) {
      const int b = cs / a.Sq;
      if (lane == 0) {
        d[0] = cu;
        d[1] = th;
        d[2] = b;
        d[3] = cL;
      }
      const int e = 32 * cc + lane;
      const bool ok = cu >= 0 && lane < 32 && e < a.topk;
      const bool any = __builtin_amdgcn_ballot_w64(ok) != 0;
      int* ring = idx_ring + (x & (W::kRing - 1)) * 32;
      if (lane < 32 && !ok) ring[lane] = -1;
      if (any ? ok : lane == 0)
        copy4_v(any ? a.indices + (size_t)cs * a.topk + e : a.seqlens, lds_addr(any ? ring : dummy));
    }
  };
  // Sparse: start the block-table lookups of item y's 32 positions.
  auto page_lookup = [&](int y) {
    if constexpr (SPARSE) {
      if (rg != 0) return;
      const int* d = desc(y);
      const int uu = __builtin_amdgcn_readfirstlane(d[0]);
      const int th = __builtin_amdgcn_readfirstlane(d[1]);
      const int bb = __builtin_amdgcn_readfirstlane(d[2]);
      const int LL = __builtin_amdgcn_readfirstlane(d[3]);
      const int ri = y & (W::kRing - 1);
      const int idx = lane < 32 ? idx_ring[ri * 32 + lane] : -1;
      const bool ok = uu >= 0 && th >= 0 && idx >= 0 && idx < LL && (idx >> 6) < a.bt_stride;
      const bool any = __builtin_amdgcn_ballot_w64(ok) != 0;
      if (any ? ok : lane == 0)
        copy4_v(any ? a.block_table + (size_t)bb * a.bt_stride + (idx >> 6) : a.seqlens,
                lds_addr(any ? pg_ring + ri * 32 : dummy));
    }
  };

  // ------------------------------------------------------------ copies
  struct Src {
    const uint8_t* base;  // dense: first row of the chunk in HBM
    const float* scales;  // dense fp8: first scale of the chunk
    int nvalid;           // dense: visible rows at the start of the chunk
    int tok;              // sparse: token (page*64 + row) of row `lane` (< 32), or -1
    i32x4 rsrc;           // dense bf16: the chunk's visible rows as a buffer resource
  };
  // Where item z's rows come from (read from its descriptor and rings).
  auto source_dense = [&](const DD& d) -> Src {
    Src r{kZeroSrc, reinterpret_cast<const float*>(kZeroSrc), 0, -1, {}};
    r.nvalid = dd_nvalid(d);
    if (r.nvalid > 0) {
      const int half = d.remh & 1;
      r.base = a.kv + (size_t)d.pg * (kPage * W::kRowBytes) + half * 32 * W::kRowBytes;
      r.scales = a.kv_scales + (size_t)d.pg * kPage + half * 32;
    }
    if constexpr (!FP8) r.rsrc = make_rsrc(r.base, (uint32_t)r.nvalid * W::kRowBytes);
    return r;
  };
  auto source = [&](int z, const Desc& dz) -> Src {
    Src r{kZeroSrc, reinterpret_cast<const float*>(kZeroSrc), 0, -1, {}};
    const int uu = dz.u, th = dz.th, LL = dz.L;
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));  // recomputed here, not kept live across the loop
      const int ri = z & (W::kRing - 1);
      const int idx = ln < 32 ? idx_ring[ri * 32 + ln] : -1;
      const int pg = ln < 32 ? pg_ring[ri * 32 + ln] : -1;
      const bool ok = uu >= 0 && th >= 0 && idx >= 0 && idx < LL && (idx >> 6) < a.bt_stride &&
                      pg >= 0 && pg < a.num_pages;
      r.tok = ok ? pg * kPage + (idx & 63) : -1;
      const unsigned m = (unsigned)__builtin_amdgcn_ballot_w64(ok);
      if (rg == 0 && ln == 0) desc(z)[4] = (int)m;
    }
    return r;
  };
  // This wave's j-th copy of an item into its blocks at LDS addresses
  // slot (region A) and slotb (region B).  Copy i = j*R + rg of an item:
  // region-A copies first, then region B, the fp8 scales, and padding.
  auto copy = [&](int j, uint32_t slot, uint32_t slotb, const Src& sr) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keeps per-lane offsets from being hoisted out of the loop
    const uint8_t* zero = kZeroSrc;
    auto rowsrc = [&](int row, uint32_t off) -> const uint8_t* {  // per-lane row
      if constexpr (!SPARSE) return row < sr.nvalid ? sr.base + row * W::kRowBytes + off : zero + off;
      else {
        const int t = __shfl(sr.tok, row);
        return t >= 0 ? a.kv + (size_t)t * W::kRowBytes + off : zero + off;
      }
    };
    const int i = j * R + rg;
    if (j < W::kNA / R) {
      if constexpr (!FP8) {  // row i, lane = 16-byte chunk position
        if constexpr (!SPARSE) {
          // rows at or past nvalid fall outside the resource and read zeros
          copy16_b(sr.rsrc, (uint32_t)(((ln ^ sw16(i)) << 4) + i * W::kRowBytes), slot + i * 1024);
        } else {
          const int t = __builtin_amdgcn_readlane(sr.tok, i);
          const uint8_t* src = t >= 0 ? a.kv + (size_t)t * W::kRowBytes : zero;
          copy16_s(src, (uint32_t)((ln ^ sw16(i)) << 4), slot + i * 1024);
        }
      } else {  // rows 2i and 2i+1, 32 lanes each
        const int row = 2 * i + (ln >> 5);
        copy16_v(rowsrc(row, (uint32_t)(((ln & 31) ^ (row & 7)) << 4)), slot + i * 1024);
      }
      return;
    }
    auto region_b = [&]() {  // RoPE parts: 8 (bf16) or 16 (fp8) rows per copy
      const int jb = i - W::kNA;
      const int row = FP8 ? 16 * jb + (ln >> 2) : 8 * jb + (ln >> 3);
      const int c = FP8 ? ((ln & 3) ^ (row & 3)) : ((ln & 7) ^ ((row >> 1) & 7));
      if constexpr (!FP8 && !SPARSE)
        copy16_b(sr.rsrc, (uint32_t)(row * W::kRowBytes + W::kABytes + (c << 4)), slotb + jb * 1024);
      else
        copy16_v(rowsrc(row, (uint32_t)(W::kABytes + (c << 4))), slotb + jb * 1024);
    };
    if constexpr (!FP8 && W::kNCopy % R == 0) {
      region_b();
    } else {
      if (i < W::kNA + W::kNB) {
        region_b();
      } else if (FP8 && i == W::kNA + W::kNB) {  // lane r < 32 copies the scale of row r
        if (ln < 32) {
          const float* src;
          if constexpr (!SPARSE) src = ln < sr.nvalid ? sr.scales + ln : reinterpret_cast<const float*>(zero);
          else src = sr.tok >= 0 ? a.kv_scales + sr.tok : reinterpret_cast<const float*>(zero);
          copy4_v(src, slotb + W::kScaleOffB);
        }
      } else if (ln == 0) {
        copy4_v(zero, lds_addr(dummy));
      }
    }
  };
  auto copy_all = [&](int z, const Src& sr) {
    const uint32_t slot = lds_addr(blk_a(z)), slotb = lds_addr(blk_b(z));
#pragma unroll
    for (int j = 0; j < W::kPerWave; j++) copy(j, slot, slotb, sr);
  };
  // Wait until this wave's copies of the item about to be computed (and
  // everything it issued before them) have landed: exactly
  // (kLeadDma - 1) steps of younger operations may stay in flight.
  auto wait_item = [&]() {
    if (rg == 0) wait_vm<(W::kLeadDma - 1) * W::per_step(0)>();
    else wait_vm<(W::kLeadDma - 1) * W::per_step(1)>();
  };
  // The prologue's copies are preceded by as many dummy lookups as a step
  // makes, so the per-step count holds from the first step on.
  auto dummy_lookups = [&]() {
    if (rg == 0 && lane == 0) {
#pragma unroll
      for (int k = 0; k < W::kLook; k++) copy4_v(a.seqlens, lds_addr(dummy));
    }
  };

  // ------------------------------------------------------------ state
  bf16x8 qf[36];
  f32x16 o[16];
  float m_run = kNegInf, l_run = 0.f;
  constexpr int DB = 16 / R;  // output dim blocks per wave
  // o[dbl * R + rb]: O^T for dims 32*(DB*rg + dbl) .., rows 32*rb + l32.

  auto load_q = [&](const UnitInfo& ui) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // as in end_segment
    const int l32 = ln & 31, g = ln >> 5;
    const int r = rg * kRowsPerWave + l32;
    const bool ok = r < ui.rows;
    const size_t grow = (size_t)ui.row0 + (ok ? r : 0);
    const bf16x8* qn = reinterpret_cast<const bf16x8*>(a.q_nope + grow * kDC + 8 * g);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(a.q_rope + grow * kDR + 8 * g);
#pragma unroll
    for (int ks = 0; ks < 32; ks++) qf[ks] = qn[2 * ks];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) qf[32 + ks] = qr[2 * ks];
    if (!ok) {
#pragma unroll
      for (int ks = 0; ks < 36; ks++) qf[ks] = bf16x8{};
    }
  };
  // Takes delivery of Q before the loop: otherwise the compiler keeps
  // waiting for these loads inside the loop, where its count cannot see the
  // copies (and would wait for all of them).
  auto take_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < 36; ks++) asm volatile("" : "+v"(qf[ks]));
  };
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < 16; i++) o[i] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;
  };

  // Per-lane pieces of the swizzled LDS addresses.
  const int ya = g ^ (FP8 ? 0 : sw16(l32));  // bf16 region A (score operand)
  const int yb = g ^ ((l32 >> 1) & 7);       // bf16 region B
  // ------------------------------------------------------------ step pieces
  // Item s lives in region-A block curA and region-B block curB; a step is
  // qk (scores, with this wave's copies of item s + kLeadDma issued between
  // the MFMAs), softmax (P and rescale factors to LDS), and after a barrier
  // rescale + pv (O += P.V).  Pipelined, the P.V of item s-1 runs beside the
  // softmax of item s instead.

  // ---- S^T[token][row] = K . Q^T over 576 dims, tokens l32 of the chunk.
  // K operands stream through a ring of kRingK registers with kLead reads
  // in flight; a register is refilled two MFMAs after its last use.
  auto qk = [&](uint32_t curA, uint32_t curB, uint32_t nxtA, uint32_t nxtB, const Src& sr) -> f32x16 {
    constexpr int kEvery = 36 / W::kPerWave;  // MFMAs between two copies
    f32x16 sacc = {};
    constexpr int kLead = 6, kRingK = 8;
    // Dense: no wait here.  A scalar load still in flight (the block table)
    // only makes the counted waits below stricter, never looser, since LDS
    // operations complete in order.
    if constexpr (SPARSE) wait_lds();
    if constexpr (!FP8) {
      uint32_t adA[8], adB[4];
#pragma unroll
      for (int k = 0; k < 8; k++) adA[k] = curA + l32 * 1024 + (((2 * k) ^ ya) << 4);
#pragma unroll
      for (int k = 0; k < 4; k++) adB[k] = curB + l32 * 128 + (((2 * k) ^ yb) << 4);
      bf16x8 ring[kRingK];
      auto rd = [&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        if constexpr (ks < 32) lds_rd16<256 * (ks >> 3)>(ring[ks % kRingK], adA[ks & 7]);
        else lds_rd16<0>(ring[ks % kRingK], adB[ks - 32]);
      };
      unroll<kLead>(rd);
      unroll<36>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        // one wait per pair of MFMAs: operands ks and ks+1 have landed
        if constexpr (ks % 2 == 0)
          lds_ready2<(kLead - 2 < 34 - ks ? kLead - 2 : 34 - ks)>(ring[ks % kRingK], ring[(ks + 1) % kRingK]);
        if constexpr (ks % kEvery == 0 && ks / kEvery < W::kPerWave) copy(ks / kEvery, nxtA, nxtB, sr);
        if constexpr (ks == 0) mfma_first(sacc, ring[0], qf[0]);
        else mfma_acc(sacc, ring[ks % kRingK], qf[ks]);
        if constexpr (ks + kLead < 36) rd(std::integral_constant<int, ks + kLead>{});
      });
      mfma_settle(sacc);
    } else {
      uint32_t adA[8], adB[4];
#pragma unroll
      for (int k = 0; k < 8; k++) adA[k] = curA + l32 * 512 + 8 * g + ((k ^ (l32 & 7)) << 4);
#pragma unroll
      for (int k = 0; k < 4; k++) adB[k] = curB + l32 * 64 + 8 * g + ((k ^ (l32 & 3)) << 4);
      u32x2 ring[kRingK];
      auto rd = [&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        if constexpr (ks < 32) lds_rd8<128 * (ks >> 3)>(ring[ks % kRingK], adA[ks & 7]);
        else lds_rd8<0>(ring[ks % kRingK], adB[ks - 32]);
      };
      unroll<kLead>(rd);
      unroll<36>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        lds_ready<(kLead - 1 < 35 - ks ? kLead - 1 : 35 - ks)>(ring[ks % kRingK]);
        if constexpr (ks % kEvery == 0 && ks / kEvery < W::kPerWave) copy(ks / kEvery, nxtA, nxtB, sr);
        const bf16x8 kf = cvt8_fp8(ring[ks % kRingK]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc, 0, 0, 0);
        if constexpr (ks + kLead < 36) rd(std::integral_constant<int, ks + kLead>{});
      });
    }
    return sacc;
  };

  // Causal masking: row r of a unit sees cached tokens below
  // rem + coff(r) of a chunk (coff = 1 + its query position - Sq);
  // without masking coff is large enough never to bind.
  int coff = 1 << 30;
  auto set_coff = [&](const UnitInfo& u) {
    if (a.causal) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      coff = 1 + (u.rin_b0 + rg * kRowsPerWave + (ln & 31)) / a.H - a.Sq;
    }
  };

  // ---- online softmax of item s: lane holds row l32, tokens
  // 8*(i/4) + 4g + i%4.  Writes P (bf16) to `pb` and the rows' rescale
  // factors to `ab`.  Dense: nv visible rows at the chunk's start, rem =
  // length - first token.  A chunk with nothing visible is computed like any
  // other: its rows are zero in LDS and every weight comes out 0.
  // fp8: token scales multiply the scores and, before P.V, the weights.
  // The row maximum is taken over the unscaled scores (the softmax scale
  // is positive) and the scale enters each weight's exponent in one FMA.
  auto softmax = [&](f32x16 sacc, const uint8_t* curB, int s, int nv, int rem, uint8_t* pb,
                     float* ab) {
    int lim = 0;
    unsigned vm = 0;
    if constexpr (!SPARSE) {
      lim = min(nv, rem + coff);
    } else {
      vm = (unsigned)__builtin_amdgcn_readfirstlane(desc(s)[4]) >> (4 * g);
    }
    const float* scl = reinterpret_cast<const float*>(curB + W::kScaleOffB) + 4 * g;
    const float c2 = a.scale_log2;
    float mloc = kNegInf;
    // Dense chunks whose 32 tokens are all visible to every row of the wave
    // (the common case) skip the masks.  Not in the pipelined kernel: there
    // the branch would split the block in which this softmax interleaves
    // with the previous chunk's P.V MFMAs (measured slower).
    bool full = false;
    if constexpr (!SPARSE && !W::kPipe) full = __builtin_amdgcn_ballot_w64(lim < 32) == 0;
    if (full) {
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        f32x4 sv = {1.f, 1.f, 1.f, 1.f};
        if constexpr (FP8) sv = *reinterpret_cast<const f32x4*>(scl + 8 * q4);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int i = 4 * q4 + e;
          if constexpr (FP8) sacc[i] *= sv[e];
          mloc = fmaxf(mloc, sacc[i]);
        }
      }
    } else {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      f32x4 sv = {1.f, 1.f, 1.f, 1.f};
      if constexpr (FP8) sv = *reinterpret_cast<const f32x4*>(scl + 8 * q4);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i = 4 * q4 + e;
        const int tau_rel = 8 * q4 + e;  // token minus 4g
        float v = sacc[i];
        bool ok;
        if constexpr (!SPARSE) ok = tau_rel + 4 * g < lim;
        else ok = (vm >> tau_rel) & 1u;
        if constexpr (FP8) v *= ok ? sv[e] : 0.f;
        sacc[i] = ok ? v : kNegInf;
        mloc = fmaxf(mloc, sacc[i]);
      }
    }
    }
    const float mt = pair_max(mloc) * c2;  // -inf stays -inf
    const float mnew = fmaxf(m_run, mt);
    const bool need = mnew > m_run + kRescaleSlack;  // -inf + slack = -inf
    const bool moved = __builtin_amdgcn_ballot_w64(need) != 0;
    // alpha is exactly 1 unless this row's maximum moved; a row with no
    // finite score yet has O = 0 and l = 0: nothing to scale.  Selects, not
    // branches, so that this code can interleave with other work.
    const float ex = __builtin_amdgcn_exp2f(m_run - mnew);
    const float alpha = (moved && m_run != kNegInf) ? ex : 1.f;
    l_run *= alpha;
    m_run = moved ? mnew : m_run;
    const float muse = (m_run == kNegInf) ? 0.f : m_run;
    float psum = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      f32x4 sv = {1.f, 1.f, 1.f, 1.f};
      if constexpr (FP8) sv = *reinterpret_cast<const f32x4*>(scl + 8 * q4);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i = 4 * q4 + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c2, -muse));
        psum += p;
        if constexpr (FP8) p *= (sacc[i] == kNegInf) ? 0.f : sv[e];
        pf[i >> 3][i & 7] = (__bf16)p;
      }
    }
    l_run += psum;

    // P row r, 16-byte chunk (g, kk) at position (2g + kk) ^ ((r >> 2) & 3).
    const int pc = (l32 >> 2) & 3;
    uint8_t* prow = pb + (32 * rg + l32) * 64;
    *reinterpret_cast<bf16x8*>(prow + (((2 * g) ^ pc) << 4)) = pf[0];
    *reinterpret_cast<bf16x8*>(prow + (((2 * g + 1) ^ pc) << 4)) = pf[1];
    ab[32 * rg + l32] = alpha;  // both halves of a row hold the same value
  };

  // ---- O *= alpha for every row whose maximum moved (rare).
  auto rescale = [&](const float* ab) {
    float al[R];
    bool scale_any = false;
#pragma unroll
    for (int rb = 0; rb < R; rb++) {
      al[rb] = ab[32 * rb + l32];
      scale_any |= al[rb] != 1.f;
    }
    if (__builtin_amdgcn_ballot_w64(scale_any) != 0) {
#pragma unroll
      for (int rb = 0; rb < R; rb++) {
#pragma unroll
        for (int dbl = 0; dbl < DB; dbl++) acc_scale(o[dbl * R + rb], al[rb]);
      }
    }
  };

  // ---- O^T[dim][row] += V^T[dim][token] . P^T[token][row] for the item
  // whose region-A block is `cur` and whose P is in `pb`; k-step kk covers
  // tokens 16kk..16kk+15 in the accumulator order of S^T.
  auto pv = [&](const uint8_t* __restrict__ cur, const uint8_t* pb) {
    // Lane offsets of the transposed V reads, recomputed here from a
    // laundered lane index so that they are not held (beside Q) through the
    // score loop, where registers are scarcest.
    int lnv = lane;
    asm volatile("" : "+v"(lnv));
    const int G16v = lnv >> 4, i16v = lnv & 15;
    const int l32v = lnv & 31, gv = lnv >> 5;
    const int pc = (l32v >> 2) & 3;
    int vbase = 0, vy0 = 0, vy1 = 0;
    int voff8[4] = {0, 0, 0, 0};
    if constexpr (!FP8) {
      // transposed reads: lane loads token 16ks + 8r + 4(G16v>>1) + (i16v>>2),
      // dims 32db + 16(G16v&1) + 4(i16v&3) .. +3
      vbase = (4 * (G16v >> 1) + (i16v >> 2)) * 1024 + 8 * (i16v & 1);
      const int w = 2 * (G16v & 1) + ((i16v >> 1) & 1);
      vy0 = w ^ (((i16v >> 2) << 2) | ((G16v >> 1) & 3));
      vy1 = w ^ (((i16v >> 2) << 2) | ((2 + (G16v >> 1)) & 3));
    } else {
      // fp8: lane loads token 16ks + 8(i16v>>3) + z8, bytes 32db + 16(G16v&1) + 8(i16v&1) .. +7
      const int z8 = 4 * (G16v >> 1) + ((i16v >> 1) & 3);
      const int trow = 8 * (i16v >> 3) + z8;
#pragma unroll
      for (int p4 = 0; p4 < 4; p4++) voff8[p4] = trow * 512 + (((2 * p4 + (G16v & 1)) ^ z8) << 4) + 8 * (i16v & 1);
    }
    auto vload = [&](int kk, int db) -> bf16x8 {
      if constexpr (!FP8) {
        const uint8_t* p0 = cur + vbase + (16 * kk) * 1024 + 256 * (db >> 2) + (((4 * (db & 3)) ^ vy0) << 4);
        const uint8_t* p1 = cur + vbase + (16 * kk + 8) * 1024 + 256 * (db >> 2) + (((4 * (db & 3)) ^ vy1) << 4);
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p0));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p1));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        const uint8_t* p = cur + voff8[db & 3] + (16 * kk) * 512 + (db >> 2) * 128;
        return cvt8_fp8(__builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(p))));
      }
    };
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      bf16x8 pbv[R], vv[DB];
#pragma unroll
      for (int rb = 0; rb < R; rb++)
        pbv[rb] = *reinterpret_cast<const bf16x8*>(pb + (32 * rb + l32v) * 64 + (((2 * gv + kk) ^ pc) << 4));
#pragma unroll
      for (int dbl = 0; dbl < DB; dbl++) vv[dbl] = vload(kk, DB * rg + dbl);
#pragma unroll
      for (int dbl = 0; dbl < DB; dbl++)
#pragma unroll
        for (int rb = 0; rb < R; rb++)
          o[dbl * R + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[dbl], pbv[rb], o[dbl * R + rb], 0, 0, 0);
    }
  };

  // ------------------------------------------------------------ epilogue
  // Normalises this wave's dims of every row and writes them to out/lse
  // (unit finished here) or to the unit's split partials.
  // The epilogue's unit eu with its cost prefix and split-index prefix,
  // walked forward as segments end (units are finished in order).
  int eu = sc.u0, eC = sc.c0, eB = sc.b0;
  auto end_segment = [&](const UnitInfo& ui, int uu) {
    // Lane-derived offsets are recomputed here rather than kept live (and
    // spilled) across the whole loop; a spill reload would wait for every
    // copy in flight.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32 = ln & 31, g = ln >> 5;
    const float lt = pair_sum(l_run);
    float* mm = mrg;
    float* ll = mrg + 32 * R;
    if constexpr (W::kPipe) {  // the merge buffers are the rescale buffers
      wait_lds();
      barrier();
    }
    if (g == 0) {
      mm[32 * rg + l32] = m_run;
      ll[32 * rg + l32] = lt;
    }
    wait_lds();
    barrier();
    for (; eu < uu; eu++) {
      const int n = unit_chunks(a, SPARSE, eu);
      int ns, gf;
      unit_splits(eC, n, sc.q, &ns, &gf);
      eC += n + kSplitCost;
      eB += ns;
    }
    int n_splits, gfirst;
    unit_splits(eC, unit_chunks(a, SPARSE, uu), sc.q, &n_splits, &gfirst);
    const int split = eB + (wg - gfirst);
#pragma unroll
    for (int rb = 0; rb < R; rb++) {
      const int r = 32 * rb + l32;
      const float mf = mm[r], lf = ll[r];
      if (r >= ui.rows) continue;
      const bool empty = !(lf > 0.f);
      const float inv = empty ? 0.f : 1.0f / lf;
      const float lse2 = empty ? kNegInf : mf + __log2f(lf);
      const bool lse_writer = g == 0 && rg == 0;
      if (n_splits <= 1) {
        uint16_t* dst = a.out + ((size_t)ui.row0 + r) * kDC + 4 * g;
#pragma unroll
        for (int dbl = 0; dbl < DB; dbl++) {
          const int db = DB * rg + dbl;
          const f32x16& ob = o[dbl * R + rb];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            bf16x2 p0 = {(__bf16)(acc_get(ob, 4 * q + 0) * inv), (__bf16)(acc_get(ob, 4 * q + 1) * inv)};
            bf16x2 p1 = {(__bf16)(acc_get(ob, 4 * q + 2) * inv), (__bf16)(acc_get(ob, 4 * q + 3) * inv)};
            u32x2 w = {__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1)};
            *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * q) = w;
          }
        }
        if (lse_writer) a.lse[(size_t)ui.row0 + r] = empty ? kNegInf : lse2 * kLn2;
      }
    }
    if (n_splits <= 1) return;
    // A split unit stores its normalised partial O/l as fp16 of O/(l M),
    // M = the row's largest |O/l| over all 512 dims (kept in fp32 beside the
    // log2 lse): the values lie in [-1, 1], so fp16 has the range, and its
    // rounding error is at most 2^-11 M, a quarter of the output's own bf16
    // rounding, for half the bytes written and read back.  The row maximum
    // is taken over the waves (each holds 512/R of the dims) through the P
    // buffers, which no wave reads any more (the barrier above).
    float* const rmax = reinterpret_cast<float*>(lds + W::kPOff);
#pragma unroll
    for (int rb = 0; rb < R; rb++) {
      const int r = 32 * rb + l32;
      float mx = 0.f;
#pragma unroll
      for (int dbl = 0; dbl < DB; dbl++)
#pragma unroll
        for (int i = 0; i < 16; i++) mx = fmaxf(mx, fabsf(acc_get(o[dbl * R + rb], i)));
      mx = pair_max(mx);
      if (g == 0) rmax[R * r + rg] = mx;
    }
    wait_lds();
    barrier();
    _Float16* const dst = reinterpret_cast<_Float16*>(a.ws_po) + (size_t)split * (32 * R * kDC) + 4 * ln;
#pragma unroll
    for (int rb = 0; rb < R; rb++) {
      const int r = 32 * rb + l32;
      if (r >= ui.rows) continue;
      const float lf = ll[r];
      const bool empty = !(lf > 0.f);
      const float inv = empty ? 0.f : 1.0f / lf;
      float mxo = 0.f;
#pragma unroll
      for (int k = 0; k < R; k++) mxo = fmaxf(mxo, rmax[R * r + k]);
      const float scale = mxo * inv;                 // the row's largest |O/l|
      const float f = scale > 0.f ? inv / scale : 0.f;
      // fragment order (see the split merge in mla_combine.hip): each store writes 512
      // consecutive bytes, 8 per lane
#pragma unroll
      for (int dbl = 0; dbl < DB; dbl++) {
        const int db = DB * rg + dbl;
        const f32x16& ob = o[dbl * R + rb];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          f16x4 w = {(_Float16)(acc_get(ob, 4 * q) * f), (_Float16)(acc_get(ob, 4 * q + 1) * f),
                     (_Float16)(acc_get(ob, 4 * q + 2) * f), (_Float16)(acc_get(ob, 4 * q + 3) * f)};
          *reinterpret_cast<f16x4*>(dst + 256 * ((rb * 16 + db) * 4 + q)) = w;
        }
      }
      if (g == 0 && rg == 0) {
        a.ws_plse[(size_t)split * (32 * R) + r] = empty ? kNegInf : mm[r] + __log2f(lf);
        a.ws_psc[(size_t)split * (32 * R) + r] = scale;
      }
    }
  };

  // ------------------------------------------------------------ prologue
  // Dense: fq[i] describes item s + i; the last entry's page load is the
  // one in flight.
  constexpr int kQ = W::kLeadDma + 2;
  DD fq[kQ];
  UnitInfo ui{};
  if constexpr (SPARSE) {
#pragma unroll 1
    for (int x = 0; x < W::kLeadCur; x++) {
      lookup(x);
      next();
    }
    wait_vm<0>();
    wait_lds();
    barrier();
#pragma unroll 1
    for (int y = 0; y < W::kLeadPage; y++) page_lookup(y);
    wait_vm<0>();
    wait_lds();
    barrier();
#pragma unroll 1
    for (int z = 0; z < W::kLeadDma; z++) {
      dummy_lookups();
      copy_all(z, source(z, read_desc(z)));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kQ; i++) {
      fq[i] = cursor_desc();
      next();
    }
    // Every workgroup starts at once, so the first requests queue behind the
    // whole opening burst: the first unit's Q goes out right after item 0's
    // copies and before the later items', and is taken before those are
    // issued, so that item 0 and Q lead the burst.
    copy_all(0, source_dense(fq[0]));
    if (fq[0].u >= 0) {
      ui = unit_info(a, false, fq[0].u);
      load_q(ui);
      take_q();
    }
#pragma unroll
    for (int z = 1; z < W::kLeadDma; z++) copy_all(z, source_dense(fq[z]));
  }

  // ------------------------------------------------------------ main loop
  // One outer iteration per unit (segment); the inner loop runs its items.
  // At a unit change the next unit's Q is requested before the finished
  // unit's results are stored, so the loads do not queue behind the stores.
  int s = 0;
  wait_item();
  wait_lds();
  barrier();
  Desc dc{}, dz{};
  if constexpr (SPARSE) {
    dc = read_desc(0);
    dz = read_desc(W::kLeadDma);
  } else {
    dc.u = fq[0].u;
  }
  int uu = dc.u;
  if constexpr (SPARSE) {
    if (uu >= 0) {
      ui = unit_info(a, SPARSE, uu);
      load_q(ui);
      take_q();
    }
  }
  // Set-up of item s at the top of its step: where the copies of item
  // s + kLeadDma come from, and (dense) the rows item s shows.
  Src sr;
  int nv = 0, rem = 0;
  DD nd{};
  auto begin_item = [&]() {
    const int z = s + W::kLeadDma;
    if constexpr (SPARSE) {
      lookup(s + W::kLeadCur);
      next();
      page_lookup(s + W::kLeadPage);
      sr = source(z, dz);
    } else {
      // Item s + kQ enters the queue at the end of this step.  Its block
      // table entry is requested here, a whole step before the queue
      // shift copies it (the copy waits for the scalar load to land).
      nd = cursor_desc();
      next();
      sr = source_dense(fq[W::kLeadDma]);
      nv = dd_nvalid(fq[0]);
      rem = fq[0].remh >> 1;
    }
  };
  auto scores = [&]() -> f32x16 {
    const int z = s + W::kLeadDma;
    f32x16 r = qk(lds_addr(blk_a(s)), lds_addr(blk_b(s)), lds_addr(blk_a(z)), lds_addr(blk_b(z)), sr);
    // In ordinary registers, so that O keeps the accumulation registers
    // while the scores wait for their softmax.
    if constexpr (W::kPipe) asm volatile("" : "+v"(r));
    return r;
  };
  auto end_item = [&]() {
    s++;
    wait_item();
    wait_lds();
    barrier();  // item s is in LDS for every wave; step s-1 is done everywhere
    if constexpr (SPARSE) {
      dc = read_desc(s);
      dz = read_desc(s + W::kLeadDma);
    } else {
#pragma unroll
      for (int i = 0; i + 1 < kQ; i++) fq[i] = fq[i + 1];
      fq[kQ - 1] = nd;
      dc.u = fq[0].u;
    }
  };
#pragma unroll 1
  while (uu >= 0) {
    reset();
    set_coff(ui);
    if constexpr (W::kPipe) {
      // The unit's first item: nothing to multiply into O yet.
      begin_item();
      softmax(scores(), blk_b(s), s, nv, rem, pbuf_of(s), alpha_of(s));
      end_item();
#pragma unroll 1
      while (dc.u == uu) {
        begin_item();
        const f32x16 sacc = scores();
        rescale(alpha_of(s - 1));
        pv(blk_a(s - 1), pbuf_of(s - 1));
        softmax(sacc, blk_b(s), s, nv, rem, pbuf_of(s), alpha_of(s));
        end_item();
      }
      // The unit's last item.
      rescale(alpha_of(s - 1));
      pv(blk_a(s - 1), pbuf_of(s - 1));
    } else {
#pragma unroll 1
      do {
        begin_item();
        softmax(scores(), blk_b(s), s, nv, rem, pbuf_of(s), alpha_of(s));
        wait_lds();
        barrier();
        rescale(alpha_of(s));
        pv(blk_a(s), pbuf_of(s));
        end_item();
      } while (dc.u == uu);
    }
    const UnitInfo done = ui;
    if (dc.u >= 0) {
      ui = unit_info(a, SPARSE, dc.u);
      load_q(ui);
    }
    end_segment(done, uu);
    wait_lds();
    barrier();  // the merge buffers are free again
    take_q();
    uu = dc.u;
  }
  wait_vm<0>();  // no copy may still be landing when the workgroup ends
}

// One entry point per (cache dtype, dense|sparse, wave shape).
#define MLA_WIDE_KERNEL(NAME, FP8, SPARSE, R)                                    \
  __global__ __launch_bounds__(64 * R, 1) void NAME(DecodeArgs a) {              \
    decode_wide<FP8, SPARSE, R>(a);                                              \
  }
MLA_WIDE_KERNEL(decode_bf16_dense_r4, false, false, 4)
MLA_WIDE_KERNEL(decode_bf16_dense_r2, false, false, 2)
MLA_WIDE_KERNEL(decode_bf16_dense_r1w, false, false, 1)
MLA_WIDE_KERNEL(decode_bf16_sparse_r1w, false, true, 1)
MLA_WIDE_KERNEL(decode_fp8_dense_r1w, true, false, 1)
MLA_WIDE_KERNEL(decode_fp8_sparse_r1w, true, true, 1)
MLA_WIDE_KERNEL(decode_bf16_sparse_r4, false, true, 4)
MLA_WIDE_KERNEL(decode_bf16_sparse_r2, false, true, 2)
MLA_WIDE_KERNEL(decode_fp8_dense_r4, true, false, 4)
MLA_WIDE_KERNEL(decode_fp8_dense_r2, true, false, 2)
MLA_WIDE_KERNEL(decode_fp8_sparse_r4, true, true, 4)
MLA_WIDE_KERNEL(decode_fp8_sparse_r2, true, true, 2)
#undef MLA_WIDE_KERNEL

template <bool FP8, bool SPARSE, int R>
hipError_t launch_wide(void (*kern)(DecodeArgs), const Geometry& g, const DecodeArgs& a,
                       hipStream_t stream) {
  using W = Wide<FP8, SPARSE, R>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, W::kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(g.num_wg), dim3(W::kThreads), W::kLdsBytes, stream, a);
  return hipGetLastError();
}

hipError_t launch_variant(bool fp8, bool sparse, const Geometry& g, const DecodeArgs& a,
                          hipStream_t s) {
  const int shape = g.m_unit > 64 ? 4 : g.m_unit > 32 ? 2 : 1;
  if (!fp8 && !sparse) {
    if (shape == 4) return launch_wide<false, false, 4>(decode_bf16_dense_r4, g, a, s);
    if (shape == 2) return launch_wide<false, false, 2>(decode_bf16_dense_r2, g, a, s);
    return launch_wide<false, false, 1>(decode_bf16_dense_r1w, g, a, s);
  }
  if (!fp8 && sparse) {
    if (shape == 4) return launch_wide<false, true, 4>(decode_bf16_sparse_r4, g, a, s);
    if (shape == 2) return launch_wide<false, true, 2>(decode_bf16_sparse_r2, g, a, s);
    return launch_wide<false, true, 1>(decode_bf16_sparse_r1w, g, a, s);
  }
  if (!sparse) {
    if (shape == 4) return launch_wide<true, false, 4>(decode_fp8_dense_r4, g, a, s);
    if (shape == 2) return launch_wide<true, false, 2>(decode_fp8_dense_r2, g, a, s);
    return launch_wide<true, false, 1>(decode_fp8_dense_r1w, g, a, s);
  }
  if (shape == 4) return launch_wide<true, true, 4>(decode_fp8_sparse_r4, g, a, s);
  if (shape == 2) return launch_wide<true, true, 2>(decode_fp8_sparse_r2, g, a, s);
  return launch_wide<true, true, 1>(decode_fp8_sparse_r1w, g, a, s);
}

}  // namespace kern

using namespace kern;

WsLayout ws_layout(const Geometry& g) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WsLayout w;
  size_t off = 0;
  w.work = off;
  off = up(off + sizeof(int32_t) * 2 * (size_t)(g.num_wg + 1));
  w.cost = off;
  off = up(off + sizeof(int32_t) * (size_t)(g.n_units + 1));
  w.meta = off;
  off = up(off + sizeof(int32_t) * 4 * (size_t)g.n_units);
  // partials: split units of the persistent kernels (fp16 values, fp32 lse
  // and scale per row), or the ranges of the head-group sparse decode (32
  // rows each, fp16 values, fp32 lse per row and scale per row and quarter
  // of the dims), whichever needs more
  size_t part_rows = (size_t)g.max_splits * g.split_rows;
  size_t sc_count = part_rows;
  if (g.sparse && g.hg_splits > 1) {
    const size_t hg_rows = (size_t)g.n_su * g.hg_groups * g.hg_splits * 32;
    if (hg_rows > part_rows) part_rows = hg_rows;
    if (4 * hg_rows > sc_count) sc_count = 4 * hg_rows;
  }
  const size_t po_bytes = sizeof(uint16_t) * part_rows * kDC;
  w.plse = off;
  off = up(off + sizeof(float) * part_rows);
  w.psc = off;
  off = up(off + sizeof(float) * sc_count);
  w.po = off;
  off = up(off + po_bytes);
  w.total = off;
  return w;
}

hipError_t launch_plan(const Geometry& g, const DecodeArgs& a, hipStream_t stream) {
  if (g.sparse)
    hipLaunchKernelGGL(plan_kernel<true>, dim3(1), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(plan_kernel<false>, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Geometry& g, const DecodeArgs& a, bool fp8, hipStream_t stream) {
  return launch_variant(fp8, g.sparse != 0, g, a, stream);
}

}  // namespace mla
