// HIP kernel of the DSA block top-k selection, written for gfx950.
//
// The sparse path attends over k << L tokens chosen per query by the
// Lightning Indexer's scores through a top-k selection on the GPU, in
// 64-token blocks ("MLA & DSA 推理性能优化指南" §1.2 figure), 16 blocks per
// query of which one initial and two local blocks always take part (§6.1
// table).  Given one indexer score per 64-token block, this kernel produces
// the token list that mla_sparse_decode consumes:
//   query s of sequence b sees L_s = L_b - Sq + s + 1 tokens, nb blocks
//   (limited to the blocks the score row covers); if nb <= n_select all are
//   taken, else blocks [0, n_init) and [nb - n_local, nb) plus the
//   n_select - n_init - n_local highest-scoring blocks between them (ties to
//   the lower block, NaN lowest); the row lists the selected blocks' token
//   positions in ascending order, -1 past L_s and in unused slots.
//
// One workgroup per query.  The middle blocks' scores become order-preserving
// 32-bit keys in LDS; a 4-pass radix select (8 bits per pass, a 256-bin LDS
// histogram each) finds the exact key T of the last block to take and how
// many blocks with key T to take; one pass over the blocks in index order
// then marks the selection (ties by their rank in index order) and compacts
// it with workgroup prefix sums, which also yields ascending order.
#include "mla_internal.h"

namespace mla {
namespace kern {
namespace {

constexpr int kSelThreads = 256;

// Larger score -> larger key; NaN counts as -inf.  -0.0 and +0.0 are the
// same score, so they get the same key (a tie, resolved by block order).
__device__ __forceinline__ unsigned score_key(float x) {
  if (x != x) x = -__builtin_inff();
  unsigned u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// Inclusive prefix sum over the workgroup's 256 threads; `total` gets the sum.
__device__ __forceinline__ int wg_incl_scan(int v, int* tmp, int& total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = wave_incl_scan(v);
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  int add = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) add += i < w ? tmp[i] : 0;
  total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return v + add;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ unsigned keys[];  // [nbk]: keys of the middle blocks
  __shared__ int hist[256];
  __shared__ int tmp[4];
  __shared__ int sel[kMaxSelect];
  __shared__ int bcast[2];
  const int tid = threadIdx.x;
  const int q = blockIdx.x;
  const int b = q / a.Sq, s = q - b * a.Sq;
  const int Ls = max(a.seqlens[b] - a.Sq + s + 1, 0);
  const int nb = min((Ls + kPage - 1) / kPage, a.nbk);
  int count;
  if (nb <= a.n_select) {
    for (int k = tid; k < nb; k += kSelThreads) sel[k] = k;
    count = nb;
  } else {
    const int lo = a.n_init, hi = nb - a.n_local, M = hi - lo;
    const int need = a.n_select - a.n_init - a.n_local;
    const float* row = a.scores + (size_t)q * a.nbk;
    for (int i = tid; i < M; i += kSelThreads) keys[i] = score_key(row[lo + i]);
    // radix select of the need-th largest key among the middle blocks
    unsigned prefix = 0, pmask = 0;
    int kk = need;
    if (need > 0) {
      for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < M; i += kSelThreads) {
          const unsigned u = keys[i];
          if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
        }
        __syncthreads();
        // thread t holds bin 255 - t: prefix sums count blocks at or above it
        const int c = hist[255 - tid];
        int tot;
        const int incl = wg_incl_scan(c, tmp, tot);
        if (incl - c < kk && kk <= incl) {
          bcast[0] = 255 - tid;
          bcast[1] = incl - c;
        }
        __syncthreads();
        prefix |= (unsigned)bcast[0] << shift;
        pmask |= 255u << shift;
        kk -= bcast[1];
        __syncthreads();
      }
    }
    const unsigned T = prefix;  // key of the last block taken (need > 0)
    const int take_ties = need > 0 ? kk : 0;
    // mark and compact in block order
    int carry_sel = 0, carry_tie = 0;
    for (int base = 0; base < nb; base += kSelThreads) {
      const int k = base + tid;
      const bool in = k < nb;
      const bool mid = in && k >= lo && k < hi;
      const unsigned key = mid ? keys[k - lo] : 0u;
      const int tie = (mid && need > 0 && key == T) ? 1 : 0;
      int tie_tot;
      const int tie_rank = carry_tie + wg_incl_scan(tie, tmp, tie_tot) - tie;
      const bool take = in && (!mid || (need > 0 && (key > T || (tie && tie_rank < take_ties))));
      const int f = take ? 1 : 0;
      int sel_tot;
      const int pos = carry_sel + wg_incl_scan(f, tmp, sel_tot) - f;
      if (take) sel[pos] = k;
      carry_tie += tie_tot;
      carry_sel += sel_tot;
    }
    count = carry_sel;
  }
  __syncthreads();
  int* out = a.indices + (size_t)q * a.n_select * kPage;
  for (int i = tid; i < a.n_select * kPage; i += kSelThreads) {
    const int j = i / kPage;
    int v = -1;
    if (j < count) {
      const int tok = sel[j] * kPage + (i % kPage);
      v = tok < Ls ? tok : -1;
    }
    out[i] = v;
  }
}

}  // namespace
}  // namespace kern

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(unsigned) * (size_t)a.nbk;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern::select_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern::select_kernel, dim3((unsigned)(a.B * a.Sq)), dim3(kern::kSelThreads), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace mla
