// Split-KV scheduling shared by the decode kernels of libmla: the units a
// decode is folded into, and the pass that partitions their 64-token tiles
// over the persistent workgroups.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace kern {

__device__ __forceinline__ int unit_tiles(const DecodeArgs& a, bool sparse, int u) {
  if (sparse) return (a.topk + kPage - 1) / kPage;
  int su = u / a.row_blocks;
  int L = ldc(a.seqlens + su);
  return L > 0 ? (L + kPage - 1) / kPage : 0;
}

struct UnitInfo {
  int b, s_fix, rows, row0, rin_b0, L;
};

__device__ __forceinline__ UnitInfo unit_info(const DecodeArgs& a, bool sparse, int u) {
  UnitInfo x;
  int su = u / a.row_blocks;
  int rb = u - su * a.row_blocks;
  x.b = sparse ? su / a.Sq : su;
  x.s_fix = sparse ? su - x.b * a.Sq : -1;
  x.rows = min(kMaxUnitRows, a.m_full - kMaxUnitRows * rb);
  x.rin_b0 = kMaxUnitRows * rb;           // first row of the unit inside its sequence unit
  x.row0 = su * a.m_full + x.rin_b0;      // flat row index of local row 0
  int L = ldc(a.seqlens + x.b);
  x.L = L > 0 ? L : 0;
  return x;
}

// ---------------------------------------------------------------------------
// Scheduler.  Cost of unit u = its tiles + kSplitCost.  Workgroup g owns the
// cost interval [g*Q, (g+1)*Q) with Q = max(ceil(total / G), kMinWgCost); a
// tile belongs to the workgroup whose interval holds its cost position.
// ---------------------------------------------------------------------------
// Units whose cost prefix fits here are searched in LDS (a binary search in
// global memory costs one memory round trip per level).
constexpr int kPlanLdsUnits = 8192;

// The scheduling pass as a device function: run by one 256-thread workgroup
// (plan_kernel, or one workgroup of a launch that also does other work).
template <bool SPARSE>
__device__ __forceinline__ void plan_work(const DecodeArgs& a) {
  __shared__ int part[256];
  __shared__ int c_lds[kPlanLdsUnits + 1];
  const int tid = threadIdx.x;
  const int U = a.n_units, G = a.num_wg;
  int32_t* C = a.ws_cost;
  const bool in_lds = U <= kPlanLdsUnits;
  const int per = (U + 255) / 256;
  const int lo = min(U, tid * per), hi = min(U, lo + per);

  int s = 0;
  for (int u = lo; u < hi; u++) s += unit_tiles(a, SPARSE, u) + kSplitCost;
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int u = lo; u < hi; u++) {
    C[u] = run;
    if (in_lds) c_lds[u] = run;
    run += unit_tiles(a, SPARSE, u) + kSplitCost;
  }
  const int total = part[255];
  if (tid == 0) {
    C[U] = total;
    if (in_lds) c_lds[U] = total;
  }
  // the zero row the main kernel copies in place of invisible cache rows
  if (tid < 1280 / 16) reinterpret_cast<i32x4*>(const_cast<uint8_t*>(a.ws_zero))[tid] = i32x4{0, 0, 0, 0};
  __threadfence_block();
  __syncthreads();

  const int Q = max((total + G - 1) / G, kMinWgCost);
  for (int g = tid; g <= G; g += 256) {
    long long x = (long long)g * Q;
    int u, t;
    if (x >= total) {
      u = U;
      t = 0;
    } else {
      const int* Cs = in_lds ? c_lds : C;
      int l = 0, h = U;  // C[l] <= x < C[h]
      while (h - l > 1) {
        int mid = (l + h) >> 1;
        if (Cs[mid] <= x) l = mid; else h = mid;
      }
      u = l;
      t = max(0, (int)(x - C[u]) - kSplitCost);
    }
    a.ws_work[2 * g] = u;
    a.ws_work[2 * g + 1] = t;
  }

  // splits per unit and their prefix
  const int* Cs = in_lds ? c_lds : C;
  int ns_sum = 0;
  for (int u = lo; u < hi; u++) {
    int n = Cs[u + 1] - Cs[u] - kSplitCost;
    int ns = 0;
    if (n > 0) {
      int gf = (Cs[u] + kSplitCost) / Q, gl = (Cs[u] + kSplitCost + n - 1) / Q;
      ns = gl - gf + 1;
    }
    ns_sum += ns;
  }
  __syncthreads();
  part[tid] = ns_sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - ns_sum;
  for (int u = lo; u < hi; u++) {
    int n = Cs[u + 1] - Cs[u] - kSplitCost;
    int ns = 0, gf = -1;
    if (n > 0) {
      gf = (Cs[u] + kSplitCost) / Q;
      int gl = (Cs[u] + kSplitCost + n - 1) / Q;
      ns = gl - gf + 1;
    }
    a.ws_meta[4 * u + 0] = n;
    a.ws_meta[4 * u + 1] = base;
    a.ws_meta[4 * u + 2] = ns;
    a.ws_meta[4 * u + 3] = gf;
    base += ns;
  }
}

}  // namespace kern
}  // namespace mla
