// C ABI of libmla: argument validation, workspace sizing and kernel launches.
// Every check runs before anything is enqueued; launches never allocate,
// free or synchronise.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "mla.h"
#include "mla_internal.h"

namespace {

thread_local char g_err[512];

mla_status fail(mla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

// Compute-unit count per device, queried once.
int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

constexpr int kMaxWg = 1 << 16;

// Folds the request into scheduling units; returns false on invalid sizes.
bool make_geometry(int B, int Sq, int H, int topk, int num_wg, mla::Geometry* g) {
  if (B <= 0 || Sq <= 0 || H <= 0 || topk < 0 || num_wg < 0 || num_wg > kMaxWg) return false;
  long long m_full = topk > 0 ? (long long)H : (long long)Sq * H;
  long long n_su = topk > 0 ? (long long)B * Sq : (long long)B;
  if (m_full > (1 << 24) || n_su > (1 << 24)) return false;
  g->B = B;
  g->Sq = Sq;
  g->H = H;
  g->sparse = topk > 0;
  g->topk = topk;
  g->n_su = (int)n_su;
  g->m_full = (int)m_full;
  g->row_blocks = (int)((m_full + mla::kMaxUnitRows - 1) / mla::kMaxUnitRows);
  long long units = n_su * g->row_blocks;
  if (units > (1 << 24)) return false;
  g->n_units = (int)units;
  g->m_unit = (int)(m_full < mla::kMaxUnitRows ? m_full : mla::kMaxUnitRows);
  g->split_rows = g->m_unit > 64 ? 128 : g->m_unit > 32 ? 64 : 32;
  g->num_wg = num_wg;
  g->max_splits = num_wg + g->n_units;
  g->hg_groups = g->hg_splits = g->hg_span = 0;
  if (g->sparse) {
    // Head-group sparse decode: items of 32 rows; an item's index list is
    // split over up to kMaxHgSplits workgroups when there are fewer items
    // than workgroups, keeping at least 16 entries per wave.
    const long long items = n_su * (((long long)H + 31) / 32);
    long long s = 1;
    if (items < num_wg && items <= mla::kMaxHgSplitItems) {
      s = (num_wg + items - 1) / items;
      const long long by_len = ((long long)topk + 63) / 64;
      if (s > by_len) s = by_len;
      if (s > mla::kMaxHgSplits) s = mla::kMaxHgSplits;
      if (s < 1) s = 1;
    }
    // entries per workgroup: a multiple of 64 (16 per wave); ranges past
    // the list's end are dropped
    const long long per_wg = ((((long long)topk + s - 1) / s) + 63) / 64 * 64;
    s = ((long long)topk + per_wg - 1) / per_wg;
    if (items * s > (1LL << 30)) return false;
    g->hg_groups = (H + 31) / 32;
    g->hg_splits = (int)s;
    g->hg_span = (int)(per_wg / 4);
  }
  return true;
}

// Workgroup count: the caller's, or one per compute unit (four for units of
// at most 32 query rows, whose one-wave workgroups share a unit).
int resolve_wg(int num_wg, int Sq, int H, int topk) {
  if (num_wg > 0) return num_wg;
  const long long rows = topk > 0 ? (long long)H : (long long)Sq * H;
  const int cus = device_cus();
  return rows <= 32 ? 4 * cus : cus;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mla_status fill_sched_args(const mla::Geometry& g, const int32_t* seqlens, void* ws,
                           mla::DecodeArgs* a) {
  mla::WsLayout w = mla::ws_layout(g);
  uint8_t* base = static_cast<uint8_t*>(ws);
  a->seqlens = seqlens;
  a->ws_work = reinterpret_cast<int32_t*>(base + w.work);
  a->ws_cost = reinterpret_cast<int32_t*>(base + w.cost);
  a->ws_meta = reinterpret_cast<int32_t*>(base + w.meta);
  a->ws_plse = reinterpret_cast<float*>(base + w.plse);
  a->ws_psc = reinterpret_cast<float*>(base + w.psc);
  a->ws_po = reinterpret_cast<float*>(base + w.po);
  a->B = g.B;
  a->Sq = g.Sq;
  a->H = g.H;
  a->topk = g.topk;
  a->n_su = g.n_su;
  a->m_full = g.m_full;
  a->row_blocks = g.row_blocks;
  a->n_units = g.n_units;
  a->num_wg = g.num_wg;
  a->split_rows = g.split_rows;
  a->hg_groups = g.hg_groups;
  a->hg_splits = g.hg_splits;
  a->hg_span = g.hg_span;
  return MLA_OK;
}

}  // namespace

// Validates a decode request and enqueues its stages (plan unless planned,
// main pass, combine) on `stream` with the given workspace.
namespace {

// Checks a decode request and folds it into its geometry and kernel
// arguments; nothing is enqueued.
mla_status prepare_decode(const void* q_nope, const void* q_rope, const void* kv_pages,
                          const float* kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                          const int32_t* block_table, int bt_stride, const int32_t* cache_seqlens,
                          const int32_t* indices, int topk, int B, int Sq, int H, float softmax_scale,
                          int causal, void* out, float* lse, void* workspace, size_t ws_bytes,
                          int num_wg, mla::Geometry* gp, mla::DecodeArgs* ap) {
  mla::Geometry& g = *gp;
  mla::DecodeArgs& a = *ap;
  if (!q_nope || !q_rope || !kv_pages || !block_table || !cache_seqlens || !out || !lse)
    return fail(MLA_ERR_NULL, "a required tensor pointer is NULL");
  if (topk > 0 && !indices) return fail(MLA_ERR_NULL, "sparse decode needs indices");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_SHAPE, "unknown kv_dtype %d", (int)kv_dtype);
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_scales)
    return fail(MLA_ERR_NULL, "fp8 cache needs kv_scales");
  if (B <= 0 || Sq <= 0 || H <= 0) return fail(MLA_ERR_SHAPE, "B, Sq, H must be >= 1 (got %d, %d, %d)", B, Sq, H);
  if (num_pages <= 0 || bt_stride <= 0)
    return fail(MLA_ERR_SHAPE, "num_pages and bt_stride must be >= 1 (got %d, %d)", num_pages, bt_stride);
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (num_wg < 0 || num_wg > kMaxWg) return fail(MLA_ERR_SHAPE, "num_wg out of range [0, %d]", kMaxWg);
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(kv_pages, 16) || !aligned(out, 16) ||
      (kv_scales && !aligned(kv_scales, 16)) || !aligned(lse, 4) || !aligned(block_table, 4) ||
      !aligned(cache_seqlens, 4) || (indices && !aligned(indices, 4)))
    return fail(MLA_ERR_ALIGN, "tensor pointer misaligned (16 B for q/kv/scales/out, 4 B for the rest)");
  if (!workspace) return fail(MLA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const int wg = resolve_wg(num_wg, Sq, H, topk);
  if (wg <= 0) return fail(MLA_ERR_HIP, "could not query the device's compute units");
  if (!make_geometry(B, Sq, H, topk, wg, &g)) return fail(MLA_ERR_SHAPE, "sizes out of range");
  const size_t need = mla::ws_layout(g).total;
  if (ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  if ((long long)num_pages * mla::kPage * mla::kD * (kv_dtype == MLA_KV_BF16 ? 2 : 1) < 0)
    return fail(MLA_ERR_SHAPE, "num_pages too large");

  memset(&a, 0, sizeof a);
  fill_sched_args(g, cache_seqlens, workspace, &a);
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.kv = static_cast<const uint8_t*>(kv_pages);
  a.kv_scales = kv_scales;
  a.block_table = block_table;
  a.indices = indices;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  a.causal = (topk == 0 && causal) ? 1 : 0;
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  return MLA_OK;
}

}  // namespace

mla_status mla::run_decode(const void* q_nope, const void* q_rope, const void* kv_pages,
                           const float* kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                           const int32_t* block_table, int bt_stride, const int32_t* cache_seqlens,
                           const int32_t* indices, int topk, int B, int Sq, int H,
                           float softmax_scale, int causal, void* out, float* lse, void* workspace,
                           size_t ws_bytes, int num_wg, int planned, hipStream_t stream, int stages) {
  g_err[0] = 0;
  mla::Geometry g;
  mla::DecodeArgs a;
  const mla_status st = prepare_decode(q_nope, q_rope, kv_pages, kv_scales, kv_dtype, num_pages, block_table,
                                       bt_stride, cache_seqlens, indices, topk, B, Sq, H, softmax_scale, causal,
                                       out, lse, workspace, ws_bytes, num_wg, &g, &a);
  if (st != MLA_OK) return st;
  hipError_t e;
  const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3;
  if (mla::uses_hg(g, fp8)) {
    // the attend stage produces finished rows: no scheduling or merge stage
    if (stages & mla::kStageAttend) {
      e = mla::launch_sparse_hg(g, a, stream);
      if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    }
    return MLA_OK;
  }
  if ((stages & mla::kStagePlan) && !planned) {
    if (g.n_units <= mla::kFoldUnits) {
      // the main pass schedules itself: one launch less
      a.fold_plan = 1;
    } else {
      e = mla::launch_plan(g, a, stream);
      if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
    }
  }
  if (stages & mla::kStageAttend) {
    e = mla::launch_decode(g, a, fp8, stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  }
  if (stages & mla::kStageCombine) {
    e = mla::launch_combine(g, a, stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  }
  return MLA_OK;
}

mla_status mla::fail_status(mla_status s, const char* msg) { return fail(s, "%s", msg); }

extern "C" {

size_t mla_workspace_size(int B, int Sq, int H, int topk, int num_wg) {
  mla::Geometry g;
  if (num_wg < 0 || num_wg > kMaxWg) return 0;
  const int wg = resolve_wg(num_wg, Sq, H, topk);
  if (wg <= 0 || !make_geometry(B, Sq, H, topk, wg, &g)) return 0;
  return mla::ws_layout(g).total;
}

mla_status mla_plan(const int32_t* cache_seqlens, int B, int Sq, int H, int topk, int num_wg,
                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (!cache_seqlens) return fail(MLA_ERR_NULL, "cache_seqlens is NULL");
  if (!workspace) return fail(MLA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(cache_seqlens, 4)) return fail(MLA_ERR_ALIGN, "cache_seqlens must be 4-byte aligned");
  if (B <= 0 || Sq <= 0 || H <= 0 || topk < 0) return fail(MLA_ERR_SHAPE, "B, Sq, H must be >= 1 and topk >= 0");
  if (num_wg < 0 || num_wg > kMaxWg) return fail(MLA_ERR_SHAPE, "num_wg out of range [0, %d]", kMaxWg);
  const int wg = resolve_wg(num_wg, Sq, H, topk);
  if (wg <= 0) return fail(MLA_ERR_HIP, "could not query the device's compute units");
  mla::Geometry g;
  if (!make_geometry(B, Sq, H, topk, wg, &g)) return fail(MLA_ERR_SHAPE, "sizes out of range");
  const size_t need = mla::ws_layout(g).total;
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  mla::DecodeArgs a;
  memset(&a, 0, sizeof a);
  fill_sched_args(g, cache_seqlens, workspace, &a);
  hipError_t e = mla::launch_plan(g, a, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status mla_decode(const void* q_nope, const void* q_rope, const void* kv_pages,
                      const float* kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                      const int32_t* block_table, int bt_stride, const int32_t* cache_seqlens,
                      int B, int Sq, int H, float softmax_scale, int causal, void* out,
                      float* lse, void* workspace, size_t ws_bytes, int num_wg, int planned,
                      hipStream_t stream) {
  return mla::run_decode(q_nope, q_rope, kv_pages, kv_scales, kv_dtype, num_pages, block_table, bt_stride,
             cache_seqlens, nullptr, 0, B, Sq, H, softmax_scale, causal, out, lse, workspace,
             ws_bytes, num_wg, planned, stream);
}

mla_status mla_sparse_decode(const void* q_nope, const void* q_rope, const void* kv_pages,
                             const float* kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                             const int32_t* block_table, int bt_stride,
                             const int32_t* cache_seqlens, const int32_t* indices, int topk,
                             int B, int Sq, int H, float softmax_scale, void* out, float* lse,
                             void* workspace, size_t ws_bytes, int num_wg, int planned,
                             hipStream_t stream) {
  g_err[0] = 0;
  if (topk <= 0) return fail(MLA_ERR_SHAPE, "topk must be >= 1 (got %d)", topk);
  return mla::run_decode(q_nope, q_rope, kv_pages, kv_scales, kv_dtype, num_pages, block_table, bt_stride,
             cache_seqlens, indices, topk, B, Sq, H, softmax_scale, 0, out, lse, workspace, ws_bytes,
             num_wg, planned, stream);
}

mla_status mla_attend(const void* q_nope, const void* q_rope, const void* kv_pages,
                      const float* kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                      const int32_t* block_table, int bt_stride, const int32_t* cache_seqlens,
                      const int32_t* indices, int topk, int B, int Sq, int H,
                      float softmax_scale, int causal, void* out, float* lse, void* workspace,
                      size_t ws_bytes, int num_wg, hipStream_t stream) {
  g_err[0] = 0;
  if (topk < 0 || (topk > 0) != (indices != nullptr))
    return fail(MLA_ERR_SHAPE, "indices and topk must be both set (sparse) or NULL and 0 (dense)");
  return mla::run_decode(q_nope, q_rope, kv_pages, kv_scales, kv_dtype, num_pages, block_table, bt_stride,
             cache_seqlens, indices, topk, B, Sq, H, softmax_scale, causal, out, lse, workspace,
             ws_bytes, num_wg, 1, stream, mla::kStageAttend);
}

mla_status mla_combine(const int32_t* cache_seqlens, int B, int Sq, int H, int topk, void* out,
                       float* lse, void* workspace, size_t ws_bytes, int num_wg,
                       hipStream_t stream) {
  g_err[0] = 0;
  if (!cache_seqlens || !out || !lse) return fail(MLA_ERR_NULL, "a required pointer is NULL");
  if (!workspace) return fail(MLA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (!aligned(out, 16) || !aligned(lse, 4) || !aligned(cache_seqlens, 4))
    return fail(MLA_ERR_ALIGN, "tensor pointer misaligned (16 B for out, 4 B for the rest)");
  if (B <= 0 || Sq <= 0 || H <= 0 || topk < 0) return fail(MLA_ERR_SHAPE, "B, Sq, H must be >= 1 and topk >= 0");
  if (num_wg < 0 || num_wg > kMaxWg) return fail(MLA_ERR_SHAPE, "num_wg out of range [0, %d]", kMaxWg);
  const int wg = resolve_wg(num_wg, Sq, H, topk);
  if (wg <= 0) return fail(MLA_ERR_HIP, "could not query the device's compute units");
  mla::Geometry g;
  if (!make_geometry(B, Sq, H, topk, wg, &g)) return fail(MLA_ERR_SHAPE, "sizes out of range");
  const size_t need = mla::ws_layout(g).total;
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  mla::DecodeArgs a;
  memset(&a, 0, sizeof a);
  fill_sched_args(g, cache_seqlens, workspace, &a);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  hipError_t e = mla::launch_combine(g, a, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

namespace {
// Layer workspace: the decode's, then q_nope and the main pass's finished
// rows (bf16 [B*Sq, H, 512] each).
struct LayerLayout {
  size_t dec, q_nope, out, total;
};
bool layer_layout(int B, int Sq, int H, int num_wg, LayerLayout* L, mla::Geometry* g) {
  const int wg = resolve_wg(num_wg, Sq, H, 0);
  if (wg <= 0 || !make_geometry(B, Sq, H, 0, wg, g)) return false;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = (size_t)B * Sq * H;
  L->dec = up(mla::ws_layout(*g).total);
  L->q_nope = L->dec;
  L->out = L->q_nope + up(rows * mla::kDC * 2);
  L->total = L->out + up(rows * mla::kDC * 2);
  return true;
}
}  // namespace

size_t mla_layer_workspace_size(int B, int Sq, int H, int num_wg) {
  if (B <= 0 || Sq <= 0 || H <= 0 || num_wg < 0 || num_wg > kMaxWg) return 0;
  if ((long long)B * Sq * H > (1LL << 31) / 512) return 0;
  LayerLayout L;
  mla::Geometry g;
  if (!layer_layout(B, Sq, H, num_wg, &L, &g)) return 0;
  return L.total;
}

mla_status mla_decode_layer(const void* q_c, const void* w_uk_t, const void* q_rope, const void* w_uv,
                            const void* kv_pages, const float* kv_scales, mla_kv_dtype kv_dtype,
                            int num_pages, const int32_t* block_table, int bt_stride,
                            const int32_t* cache_seqlens, int B, int Sq, int H, float softmax_scale,
                            int causal, void* o, float* lse, void* workspace, size_t ws_bytes,
                            int num_wg, hipStream_t stream) {
  g_err[0] = 0;
  if (!q_c || !w_uk_t || !w_uv || !o) return fail(MLA_ERR_NULL, "a required tensor pointer is NULL");
  if (!aligned(q_c, 16) || !aligned(w_uk_t, 16) || !aligned(w_uv, 16) || !aligned(o, 16))
    return fail(MLA_ERR_ALIGN, "q_c, w_uk_t, w_uv and o must be 16-byte aligned");
  if (B <= 0 || Sq <= 0 || H <= 0 || H > 65535)
    return fail(MLA_ERR_SHAPE, "need B, Sq >= 1 and 1 <= H <= 65535 (got %d, %d, %d)", B, Sq, H);
  if ((long long)B * Sq * H > (1LL << 31) / 512) return fail(MLA_ERR_SHAPE, "B * Sq * H too large");
  if (num_wg < 0 || num_wg > kMaxWg) return fail(MLA_ERR_SHAPE, "num_wg out of range [0, %d]", kMaxWg);
  if (!workspace) return fail(MLA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  LayerLayout L;
  mla::Geometry g0;
  if (!layer_layout(B, Sq, H, num_wg, &L, &g0)) return fail(MLA_ERR_SHAPE, "sizes out of range");
  if (ws_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  mla::LayerArgs la;
  memset(&la, 0, sizeof la);
  mla::Geometry g;
  const mla_status st = prepare_decode(base + L.q_nope, q_rope, kv_pages, kv_scales, kv_dtype, num_pages,
                                       block_table, bt_stride, cache_seqlens, nullptr, 0, B, Sq, H,
                                       softmax_scale, causal, base + L.out, lse, workspace, L.dec, num_wg,
                                       &g, &la.d);
  if (st != MLA_OK) return st;
  la.pa.a = static_cast<const uint16_t*>(q_c);
  la.pa.w = static_cast<const uint16_t*>(w_uk_t);
  la.pa.c = reinterpret_cast<uint16_t*>(base + L.q_nope);
  la.pa.M = B * Sq;
  la.pa.H = H;
  mla::ProjArgs pj;
  pj.a = reinterpret_cast<const uint16_t*>(base + L.out);
  pj.w = static_cast<const uint16_t*>(w_uv);
  pj.c = static_cast<uint16_t*>(o);
  pj.M = B * Sq;
  pj.H = H;
  // Up to kFoldUnits units the main pass schedules itself and the absorption
  // is the plain GEMM; beyond, the schedule rides in the absorption launch.
  hipError_t e;
  if (g.n_units <= mla::kFoldUnits) {
    la.d.fold_plan = 1;
    e = mla::launch_proj(la.pa, true, stream);
  } else {
    e = mla::launch_absorb_plan(la, stream);
  }
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "absorb launch: %s", hipGetErrorString(e));
  e = mla::launch_decode(g, la.d, kv_dtype == MLA_KV_FP8_E4M3, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  e = mla::launch_combine(g, la.d, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  e = mla::launch_proj(pj, false, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status mla_kv_append(const void* new_kv, void* kv_pages, float* kv_scales,
                         mla_kv_dtype kv_dtype, int num_pages, const int32_t* block_table,
                         int bt_stride, const int32_t* cache_seqlens, int B, int Sq,
                         hipStream_t stream) {
  g_err[0] = 0;
  if (!new_kv || !kv_pages || !block_table || !cache_seqlens)
    return fail(MLA_ERR_NULL, "a required tensor pointer is NULL");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_SHAPE, "unknown kv_dtype %d", (int)kv_dtype);
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_scales) return fail(MLA_ERR_NULL, "fp8 cache needs kv_scales");
  if (B <= 0 || Sq <= 0) return fail(MLA_ERR_SHAPE, "B, Sq must be >= 1 (got %d, %d)", B, Sq);
  if ((long long)B * Sq > (1LL << 30)) return fail(MLA_ERR_SHAPE, "B * Sq too large");
  if (num_pages <= 0 || bt_stride <= 0)
    return fail(MLA_ERR_SHAPE, "num_pages and bt_stride must be >= 1 (got %d, %d)", num_pages, bt_stride);
  if (!aligned(new_kv, 16) || !aligned(kv_pages, 16) || (kv_scales && !aligned(kv_scales, 4)) ||
      !aligned(block_table, 4) || !aligned(cache_seqlens, 4))
    return fail(MLA_ERR_ALIGN, "tensor pointer misaligned (16 B for new_kv/kv, 4 B for the rest)");
  mla::AppendArgs a;
  a.src = static_cast<const uint16_t*>(new_kv);
  a.kv = static_cast<uint8_t*>(kv_pages);
  a.kv_scales = kv_scales;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.B = B;
  a.Sq = Sq;
  a.bt_stride = bt_stride;
  a.num_pages = num_pages;
  hipError_t e = mla::launch_append(a, kv_dtype == MLA_KV_FP8_E4M3, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status mla_dsa_select(const float* block_scores, int nbk, const int32_t* cache_seqlens, int B,
                          int Sq, int n_select, int n_init, int n_local, int32_t* indices,
                          hipStream_t stream) {
  g_err[0] = 0;
  if (!block_scores || !cache_seqlens || !indices)
    return fail(MLA_ERR_NULL, "a required tensor pointer is NULL");
  if (B <= 0 || Sq <= 0) return fail(MLA_ERR_SHAPE, "B, Sq must be >= 1 (got %d, %d)", B, Sq);
  if ((long long)B * Sq > (1LL << 30)) return fail(MLA_ERR_SHAPE, "B * Sq too large");
  if (nbk <= 0) return fail(MLA_ERR_SHAPE, "nbk must be >= 1 (got %d)", nbk);
  if (nbk > mla::kMaxSelBlocks)
    return fail(MLA_ERR_UNSUPPORTED, "nbk %d exceeds %d blocks per score row", nbk, mla::kMaxSelBlocks);
  if (n_select <= 0 || n_select > mla::kMaxSelect)
    return fail(MLA_ERR_SHAPE, "n_select must be in [1, %d] (got %d)", mla::kMaxSelect, n_select);
  if (n_init < 0 || n_local < 0 || n_init + n_local > n_select)
    return fail(MLA_ERR_SHAPE, "n_init, n_local must be >= 0 with n_init + n_local <= n_select");
  if (!aligned(block_scores, 4) || !aligned(cache_seqlens, 4) || !aligned(indices, 4))
    return fail(MLA_ERR_ALIGN, "tensor pointers must be 4-byte aligned");
  mla::SelectArgs a;
  a.scores = block_scores;
  a.seqlens = cache_seqlens;
  a.indices = indices;
  a.B = B;
  a.Sq = Sq;
  a.nbk = nbk;
  a.n_select = n_select;
  a.n_init = n_init;
  a.n_local = n_local;
  hipError_t e = mla::launch_select(a, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "select launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

namespace {
mla_status run_proj(const void* act, const void* w, void* c, int M, int H, bool absorb,
                    hipStream_t stream) {
  g_err[0] = 0;
  if (!act || !w || !c) return fail(MLA_ERR_NULL, "a required tensor pointer is NULL");
  if (M <= 0 || H <= 0 || H > 65535) return fail(MLA_ERR_SHAPE, "need M >= 1 and 1 <= H <= 65535 (got %d, %d)", M, H);
  if ((long long)M * H > (1LL << 31) / 512) return fail(MLA_ERR_SHAPE, "M * H too large");
  if (!aligned(act, 16) || !aligned(w, 16) || !aligned(c, 16))
    return fail(MLA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  mla::ProjArgs a;
  a.a = static_cast<const uint16_t*>(act);
  a.w = static_cast<const uint16_t*>(w);
  a.c = static_cast<uint16_t*>(c);
  a.M = M;
  a.H = H;
  hipError_t e = mla::launch_proj(a, absorb, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return MLA_OK;
}
}  // namespace

mla_status mla_absorb_query(const void* q_c, const void* w_uk_t, void* q_nope, int M, int H,
                            hipStream_t stream) {
  return run_proj(q_c, w_uk_t, q_nope, M, H, true, stream);
}

mla_status mla_project_out(const void* out_latent, const void* w_uv, void* o, int M, int H,
                           hipStream_t stream) {
  return run_proj(out_latent, w_uv, o, M, H, false, stream);
}

mla_status mla_prefill(const void* q, const void* k, const void* v, int B, int T, int H,
                       float softmax_scale, int causal, void* out, float* lse, hipStream_t stream) {
  g_err[0] = 0;
  if (!q || !k || !v || !out || !lse) return fail(MLA_ERR_NULL, "a required tensor pointer is NULL");
  if (B <= 0 || T <= 0 || H <= 0 || H > 65535 || B > 65535)
    return fail(MLA_ERR_SHAPE, "need B, T >= 1 and 1 <= H, B <= 65535 (got %d, %d, %d)", B, T, H);
  if ((long long)B * T * H > (1LL << 31) / 192 || (long long)(T + 64) * H * 384 > (1LL << 32))
    return fail(MLA_ERR_SHAPE, "B * T * H or T * H too large");
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(MLA_ERR_ALIGN, "tensor pointer misaligned (16 B for q/k/v/out, 4 B for lse)");
  mla::PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = B;
  a.T = T;
  a.H = H;
  a.causal = causal ? 1 : 0;
  a.scale = softmax_scale;
  hipError_t e = mla::launch_prefill(a, stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return MLA_OK;
}

const char* mla_status_str(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_err; }

}  // extern "C"
