// Split-KV merge for the persistent decode kernels, for gfx950.
//
// A unit (up to 128 query rows of one sequence) whose tiles were spread over
// several workgroups leaves one partial result per split: the normalised
// output O/l and the log-sum-exp of its scores.  "MLA 最佳算子全景调研" §2-§3
// (split-KV with a combine step) merges them by their log-sum-exp:
//   lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * (O/l)_s.
// Units with no visible token at all get out = 0 and lse = -inf.
//
// Partial layout per split (32 * R rows, R the waves of the main kernel's
// shape): 64 * R blocks of 256 fp16 in fragment order.  Block
// (rb, db, q) = (rb * 16 + db) * 4 + q holds, at lane L = 32 g + l (four
// values, 8 bytes), row 32 rb + l, dims 32 db + 8 q + 4 g .. +3, divided by
// the row's scale: the order in which a wave's accumulators leave the
// registers.  Per split and row: the log2 lse and the scale (fp32).
//
// The merge is bound by HBM: every partial byte is read once.  A thread
// takes 16 consecutive bytes of a fragment block (lanes 2 j and 2 j + 1:
// rows 32 rb + 2 (j & 15) and the next, dims 32 db + 8 q + 4 (j >> 4) .. +3)
// and keeps the loads of four splits in flight (16 bytes of lse and scale
// and 16 of values each).  When a unit can be expected to have many splits
// (a few long sequences over all workgroups), 4 or 8 thread groups share its
// splits out and merge their states through LDS.
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {
namespace kern {

// kBatch: splits whose loads a thread keeps in flight together (4, or 8
// when its group can be expected to walk at least 8 splits).
template <bool SPARSE, int SG, int kBatch>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  // Flat grid, a unit's blocks consecutive, so that blocks dispatched
  // together read consecutive 4 KB of the same partials.  A block covers F
  // fragment blocks; its SG = 8 / F thread groups take the unit's splits in
  // turn (group g: splits g, g + SG, ...) and are merged through LDS.
  constexpr int F = 8 / SG;
  const int per_unit = gridDim.x / a.n_units;
  const int uu = blockIdx.x / per_unit, by = blockIdx.x - uu * per_unit;
  const int ns = a.ws_meta[4 * uu + 2];
  if (ns == 1) return;  // uniform: the unit was finished by one workgroup
  const int t = threadIdx.x;
  const int fl = (t >> 5) % F, sg = (t >> 5) / F;
  const int blk = by * F + fl;  // fragment block (rb, db, q)
  const int j = t & 31;
  const int q = blk & 3, db = (blk >> 2) & 15, rb = blk >> 6;
  const int r = 32 * rb + 2 * (j & 15);       // first of the two rows
  const UnitInfo ui = unit_info(a, SPARSE, uu);
  const bool active = r < ui.rows;
  const bool second = r + 1 < ui.rows;
  const int d4 = 32 * db + 8 * q + 4 * (j >> 4);
  const size_t grow = (size_t)ui.row0 + r;
  uint16_t* const dst = a.out + grow * kDC + d4;
  const bool lse_writer = db == 0 && q == 0 && j < 16;
  if (ns == 0) {  // uniform: no visible token in the whole unit
    if (active && sg == 0) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{0u, 0u};
      if (second) *reinterpret_cast<u32x2*>(dst + kDC) = u32x2{0u, 0u};
      if (lse_writer) {
        a.lse[grow] = kNegInf;
        if (second) a.lse[grow + 1] = kNegInf;
      }
    }
    return;
  }
  const int base = a.ws_meta[4 * uu + 1];
  const size_t split_elems = (size_t)a.split_rows * kDC;
  const _Float16* const po = reinterpret_cast<const _Float16*>(a.ws_po) + (size_t)blk * 256 + 8 * j;
  const float* const plse = a.ws_plse + r;
  const float* const psc = a.ws_psc + r;

  // running (max, sum of weights, weighted values) of the two rows over this
  // group's splits
  float mx0 = kNegInf, mx1 = kNegInf, ws0 = 0.f, ws1 = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = sg; active && i0 < ns; i0 += SG * kBatch) {
    float2 ls[kBatch], sc[kBatch];
    f16x8 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; k++) {
      // past the last split no load (the same for the whole thread group);
      // padding has lse -inf, so weight 0
      const int s = i0 + k * SG;
      if (s < ns) {
        const size_t sp = (size_t)(base + s);
        ls[k] = *reinterpret_cast<const float2*>(plse + sp * a.split_rows);
        sc[k] = *reinterpret_cast<const float2*>(psc + sp * a.split_rows);
        v[k] = *reinterpret_cast<const f16x8*>(po + sp * split_elems);
      } else {
        ls[k] = float2{kNegInf, kNegInf};
        sc[k] = float2{0.f, 0.f};
        v[k] = f16x8{};
      }
    }
    float bm0 = mx0, bm1 = mx1;
#pragma unroll
    for (int k = 0; k < kBatch; k++) {
      bm0 = fmaxf(bm0, ls[k].x);
      bm1 = fmaxf(bm1, ls[k].y);
    }
    // rescale what was merged so far to the batch's maximum (0 while the
    // row has seen nothing; a row still at -inf stays as it is)
    const float r0 = bm0 == kNegInf ? 1.f : __builtin_amdgcn_exp2f(mx0 - bm0);
    const float r1 = bm1 == kNegInf ? 1.f : __builtin_amdgcn_exp2f(mx1 - bm1);
    acc0 *= r0;
    acc1 *= r1;
    ws0 *= r0;
    ws1 *= r1;
    mx0 = bm0;
    mx1 = bm1;
#pragma unroll
    for (int k = 0; k < kBatch; k++) {
      // weight 0 for an empty split (lse -inf) and for padding
      const float w0 = bm0 != kNegInf ? __builtin_amdgcn_exp2f(ls[k].x - bm0) : 0.f;
      const float w1 = bm1 != kNegInf ? __builtin_amdgcn_exp2f(ls[k].y - bm1) : 0.f;
      ws0 += w0;
      ws1 += w1;
      const float f0 = w0 * sc[k].x, f1 = w1 * sc[k].y;
      // an empty split's values may be anything finite; its weight is 0
      // (values 0..3: lane 2 j, the first row; 4..7: lane 2 j + 1)
      acc0 += f0 * f32x4{(float)v[k][0], (float)v[k][1], (float)v[k][2], (float)v[k][3]};
      acc1 += f1 * f32x4{(float)v[k][4], (float)v[k][5], (float)v[k][6], (float)v[k][7]};
    }
  }
  if constexpr (SG > 1) {
    // each group's state at [sg][fl][j]; group 0 merges the others into its
    // own by the same log-sum-exp rule, in group order
    __shared__ float st[12][256];
    const int e = (sg * F + fl) * 32 + j;
    st[0][e] = mx0;
    st[1][e] = mx1;
    st[2][e] = ws0;
    st[3][e] = ws1;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      st[4 + c][e] = acc0[c];
      st[8 + c][e] = acc1[c];
    }
    __syncthreads();
    if (sg != 0) return;
    for (int g2 = 1; g2 < SG; g2++) {
      const int f = (g2 * F + fl) * 32 + j;
      const float m0 = st[0][f], m1 = st[1][f];
      const float n0 = fmaxf(mx0, m0), n1 = fmaxf(mx1, m1);
      const float a0 = n0 == kNegInf ? 1.f : __builtin_amdgcn_exp2f(mx0 - n0);
      const float a1 = n1 == kNegInf ? 1.f : __builtin_amdgcn_exp2f(mx1 - n1);
      const float b0 = n0 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m0 - n0);
      const float b1 = n1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m1 - n1);
      ws0 = ws0 * a0 + st[2][f] * b0;
      ws1 = ws1 * a1 + st[3][f] * b1;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        acc0[c] = acc0[c] * a0 + st[4 + c][f] * b0;
        acc1[c] = acc1[c] * a1 + st[8 + c][f] * b1;
      }
      mx0 = n0;
      mx1 = n1;
    }
  }
  if (!active) return;
  auto put = [&](uint16_t* p, const f32x4& acc, float wsum, float mx, size_t row) {
    if (mx == kNegInf) {
      *reinterpret_cast<u32x2*>(p) = u32x2{0u, 0u};
      if (lse_writer) a.lse[row] = kNegInf;
      return;
    }
    const float inv = 1.0f / wsum;
    const bf16x2 p0 = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
    const bf16x2 p1 = {(__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)};
    *reinterpret_cast<u32x2*>(p) = u32x2{__builtin_bit_cast(unsigned, p0), __builtin_bit_cast(unsigned, p1)};
    if (lse_writer) a.lse[row] = (mx + __log2f(wsum)) * kLn2;
  };
  put(dst, acc0, ws0, mx0, grow);
  if (second) put(dst + kDC, acc1, ws1, mx1, grow + 1);
}

}  // namespace kern

hipError_t launch_combine(const Geometry& g, const DecodeArgs& a, hipStream_t stream) {
  // Thread groups per unit from the splits a unit can be expected to have
  // (the workgroups shared over the units, plus one): a long chain of splits
  // is shared out among the groups instead of walked by each thread alone
  // (up to 16 splits one group measured faster); 8 loads in flight per
  // thread when its group can be expected to walk 8 splits or more.
  const int est = (g.num_wg + g.n_units - 1) / g.n_units + 1;
  const int sg = est > 32 ? 8 : est > 16 ? 4 : 1;
  const bool deep = est >= 8 * sg;
  // a unit has 64 fragment blocks (4 KB of fp16 each) per 32 rows; a
  // 256-thread block covers 8 / sg of them
  const dim3 grid((unsigned)g.n_units * (unsigned)(((g.m_unit + 31) / 32) * 8 * sg));
  auto go = [&](auto SPARSE, auto SG) {
    constexpr bool sp = decltype(SPARSE)::value;
    constexpr int gs = decltype(SG)::value;
    if (deep)
      hipLaunchKernelGGL((kern::combine_kernel<sp, gs, 8>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((kern::combine_kernel<sp, gs, 4>), grid, dim3(256), 0, stream, a);
  };
  auto by_groups = [&](auto SPARSE) {
    if (sg == 8) go(SPARSE, std::integral_constant<int, 8>{});
    else if (sg == 4) go(SPARSE, std::integral_constant<int, 4>{});
    else go(SPARSE, std::integral_constant<int, 1>{});
  };
  if (g.sparse) by_groups(std::true_type{});
  else by_groups(std::false_type{});
  return hipGetLastError();
}

}  // namespace mla
