// Split-KV scheduling shared by the decode kernels of libmla: the units a
// decode is folded into, and the pass that partitions their 32-token chunks
// (half pages) over the persistent workgroups.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace kern {

// A unit's 32-token chunks, at most (2^31 - 2^17) / n_units - kSplitCost of
// them, so that the schedule's 32-bit cost arithmetic (the prefix plus up to
// 2^16 workgroups) cannot overflow whatever lengths the caller passes (the
// bound is past 6e10 tokens in all).
__device__ __forceinline__ int unit_chunks(const DecodeArgs& a, bool sparse, int u) {
  const int cap = (0x7fffffff - (1 << 17)) / a.n_units - kSplitCost;
  if (sparse) return min((a.topk - 1) / 32 + 1, cap);
  int su = u / a.row_blocks;
  int L = ldc(a.seqlens + su);
  return L > 0 ? min((L - 1) / 32 + 1, cap) : 0;
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
// Scheduler.  Cost of unit u = its chunks + kSplitCost.  Workgroup g owns
// the cost interval [g*Q, (g+1)*Q) with Q = max(ceil(total / G), kMinWgCost);
// a chunk belongs to the workgroup whose interval holds its cost position.
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
  for (int u = lo; u < hi; u++) s += unit_chunks(a, SPARSE, u) + kSplitCost;
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
    run += unit_chunks(a, SPARSE, u) + kSplitCost;
  }
  const int total = part[255];
  if (tid == 0) {
    C[U] = total;
    if (in_lds) c_lds[U] = total;
  }
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

// What one workgroup of the main pass needs of the schedule: its first and
// last (unit, chunk) -- [u0, t0) up to (u1, t1), chunks of u1 below t1 -- the
// cost quantum q, and the cost prefix c0 and split-index prefix b0 at its
// first unit; later units' values follow from these by walking the units in
// order (split_of).
struct WgSched {
  int u0, t0, u1, t1, q, c0, b0;
};

// Splits of a unit of n chunks whose cost interval starts at c, and the
// first workgroup that holds one (-1 for a unit with no chunk).
__device__ __forceinline__ void unit_splits(int c, int n, int q, int* ns, int* gf) {
  if (n <= 0) {
    *ns = 0;
    *gf = -1;
    return;
  }
  *gf = (c + kSplitCost) / q;
  *ns = (c + kSplitCost + n - 1) / q - *gf + 1;
}

// Inclusive prefix sum of x over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Units the main pass schedules for itself (up to kFoldUnits), in the LDS
// it has not started using yet (2 (U + 1) ints), instead of reading a
// separate scheduling launch's output: every workgroup computes the same
// cost prefix and finds its own share, and the workgroup whose share holds
// a unit's cost position writes that unit's metadata for the split merge.
// Wave 0 does the prefix sums with lane shuffles (each lane takes a run of
// consecutive units), so the other waves wait at a single barrier.
template <bool SPARSE>
__device__ WgSched sched_in_wg(const DecodeArgs& a, int* scr, int tid, int wg) {
  const int U = a.n_units, G = a.num_wg;
  int* const C = scr;           // [U + 1] cost prefix
  int* const NS = C + U + 1;    // [U + 1] prefix of split counts
  if (tid < 64) {
    const int lane = tid;
    const int per = (U + 63) / 64;
    const int lo = min(U, lane * per), hi = min(U, lo + per);
    int s = 0;
    for (int u = lo; u < hi; u++) s += unit_chunks(a, SPARSE, u) + kSplitCost;
    const int incl = wave_incl_scan(s, lane);
    const int total = __shfl(incl, 63, 64);
    int run = incl - s;
    for (int u = lo; u < hi; u++) {
      C[u] = run;
      run += unit_chunks(a, SPARSE, u) + kSplitCost;
    }
    if (lane == 63) C[U] = total;
    const int q = max((total + G - 1) / G, kMinWgCost);
    int ns_sum = 0;
    for (int u = lo; u < hi; u++) {
      int ns, gf;
      unit_splits(C[u], C[u + 1] - C[u] - kSplitCost, q, &ns, &gf);
      ns_sum += ns;
    }
    const int ns_incl = wave_incl_scan(ns_sum, lane);
    int base = ns_incl - ns_sum;
    for (int u = lo; u < hi; u++) {
      const int n = C[u + 1] - C[u] - kSplitCost;
      int ns, gf;
      unit_splits(C[u], n, q, &ns, &gf);
      NS[u] = base;
      if (C[u] / q == wg) {  // one writer per unit
        a.ws_meta[4 * u + 0] = n;
        a.ws_meta[4 * u + 1] = base;
        a.ws_meta[4 * u + 2] = ns;
        a.ws_meta[4 * u + 3] = gf;
      }
      base += ns;
    }
    if (lane == 63) NS[U] = ns_incl;
  }
  __syncthreads();
  const int total = C[U];
  const int q = max((total + G - 1) / G, kMinWgCost);
  // this workgroup's share [wg q, (wg + 1) q) of the cost line
  auto locate = [&](long long x, int* u, int* t) {
    if (x >= total) {
      *u = U;
      *t = 0;
      return;
    }
    int l = 0, h = U;  // C[l] <= x < C[h]
    while (h - l > 1) {
      const int mid = (l + h) >> 1;
      if (C[mid] <= x) l = mid; else h = mid;
    }
    *u = l;
    *t = max(0, (int)(x - C[l]) - kSplitCost);
  };
  WgSched w;
  locate((long long)wg * q, &w.u0, &w.t0);
  locate((long long)(wg + 1) * q, &w.u1, &w.t1);
  w.q = q;
  w.c0 = C[min(w.u0, U)];
  w.b0 = NS[min(w.u0, U)];
  w.u0 = __builtin_amdgcn_readfirstlane(w.u0);
  w.t0 = __builtin_amdgcn_readfirstlane(w.t0);
  w.u1 = __builtin_amdgcn_readfirstlane(w.u1);
  w.t1 = __builtin_amdgcn_readfirstlane(w.t1);
  w.q = __builtin_amdgcn_readfirstlane(w.q);
  w.c0 = __builtin_amdgcn_readfirstlane(w.c0);
  w.b0 = __builtin_amdgcn_readfirstlane(w.b0);
  __syncthreads();  // the scratch is the LDS ring: free it for the copies
  return w;
}

}  // namespace kern
}  // namespace mla
