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
// and 16 of values each).
#include "mla_device.h"
#include "mla_internal.h"
#include "mla_sched.h"

namespace mla {
namespace kern {

namespace {
constexpr int kBatch = 4;  // splits whose loads are in flight together (8 and 16 measured slower)
}

template <bool SPARSE>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  // flat grid: consecutive blocks take consecutive 4 KB of one unit's partials
  const int per_unit = gridDim.x / a.n_units;
  const int uu = blockIdx.x / per_unit, by = blockIdx.x - uu * per_unit;
  const int ns = a.ws_meta[4 * uu + 2];
  if (ns == 1) return;
  const int t = threadIdx.x;
  const int blk = by * 8 + (t >> 5);  // fragment block (rb, db, q)
  const int j = t & 31;
  const int q = blk & 3, db = (blk >> 2) & 15, rb = blk >> 6;
  const int r = 32 * rb + 2 * (j & 15);       // first of the two rows
  const UnitInfo ui = unit_info(a, SPARSE, uu);
  if (r >= ui.rows) return;
  const bool second = r + 1 < ui.rows;
  const int d4 = 32 * db + 8 * q + 4 * (j >> 4);
  const size_t grow = (size_t)ui.row0 + r;
  uint16_t* const dst = a.out + grow * kDC + d4;
  const bool lse_writer = db == 0 && q == 0 && j < 16;
  if (ns == 0) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{0u, 0u};
    if (second) *reinterpret_cast<u32x2*>(dst + kDC) = u32x2{0u, 0u};
    if (lse_writer) {
      a.lse[grow] = kNegInf;
      if (second) a.lse[grow + 1] = kNegInf;
    }
    return;
  }
  const int base = a.ws_meta[4 * uu + 1];
  const size_t split_elems = (size_t)a.split_rows * kDC;
  const _Float16* const po = reinterpret_cast<const _Float16*>(a.ws_po) + (size_t)blk * 256 + 8 * j;
  const float* const plse = a.ws_plse + r;
  const float* const psc = a.ws_psc + r;

  // running (max, sum of weights, weighted values) of the two rows
  float mx0 = kNegInf, mx1 = kNegInf, ws0 = 0.f, ws1 = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < ns; i0 += kBatch) {
    float2 ls[kBatch], sc[kBatch];
    f16x8 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; k++) {
      // ns is the same for the whole block: past the last split no load
      if (i0 + k < ns) {
        const size_t sp = (size_t)(base + i0 + k);
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
      if (i0 + k < ns) {
        bm0 = fmaxf(bm0, ls[k].x);
        bm1 = fmaxf(bm1, ls[k].y);
      }
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
      const bool in = i0 + k < ns;
      // weight 0 for an empty split (lse -inf) and for padding
      const float w0 = (in && bm0 != kNegInf) ? __builtin_amdgcn_exp2f(ls[k].x - bm0) : 0.f;
      const float w1 = (in && bm1 != kNegInf) ? __builtin_amdgcn_exp2f(ls[k].y - bm1) : 0.f;
      ws0 += w0;
      ws1 += w1;
      const float f0 = w0 * sc[k].x, f1 = w1 * sc[k].y;
      // an empty split's values may be anything finite; its weight is 0
      // (values 0..3: lane 2 j, the first row; 4..7: lane 2 j + 1)
      acc0 += f0 * f32x4{(float)v[k][0], (float)v[k][1], (float)v[k][2], (float)v[k][3]};
      acc1 += f1 * f32x4{(float)v[k][4], (float)v[k][5], (float)v[k][6], (float)v[k][7]};
    }
  }
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
  // 8 fragment blocks (4 KB of fp16) per 256-thread block, 64 per 32 rows
  dim3 grid((unsigned)g.n_units * (unsigned)(((g.m_unit + 31) / 32) * 8));
  if (g.sparse)
    hipLaunchKernelGGL(kern::combine_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kern::combine_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
