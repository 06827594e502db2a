// Internal declarations shared by the kernels and the C-ABI layer of libmla.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

constexpr int kDC = 512;             // latent dims (value part)
constexpr int kDR = 64;              // RoPE key dims
constexpr int kD = kDC + kDR;        // 576 cached dims per token
constexpr int kPage = 64;            // tokens per page == tokens per tile
constexpr int kRowsPerWave = 32;     // query rows one wave owns
constexpr int kMaxUnitRows = 128;    // query rows per scheduling unit
constexpr int kBytesBf16Row = kD * 2;   // 1152
constexpr int kBytesFp8Row = kD;        // 576
constexpr int kTileBf16 = kPage * kBytesBf16Row;  // 73728
constexpr int kTileFp8 = kPage * kBytesFp8Row;    // 36864

// Scheduling constants, in 32-token chunks (the unit of work of the main
// pass): a split costs this many chunks of fixed work (its query load, its
// first chunk without the pipeline, its partial written and read back; 8
// measured best of 5 to 12), and the least work a workgroup is given (one
// chunk: a small decode is spread over as many workgroups as it has chunks).
constexpr int kSplitCost = 8;
constexpr int kMinWgCost = 1;
// Decodes of up to this many units schedule themselves inside the main pass
// (its LDS holds the cost prefix); larger ones get a scheduling launch.
constexpr int kFoldUnits = 2048;

// Problem geometry after the host has folded (B, Sq, H, sparse) into units.
// A "sequence unit" (su) is a set of query rows that attend over the same
// tokens: dense -> one per batch entry (Sq*H rows); sparse -> one per
// (b, s) (H rows).  Units split a sequence unit into blocks of <= 128 rows.
struct Geometry {
  int B, Sq, H;
  int sparse, topk;
  int n_su;        // sequence units
  int m_full;      // rows per sequence unit
  int row_blocks;  // ceil(m_full / 128)
  int n_units;     // n_su * row_blocks
  int m_unit;      // min(m_full, 128): selects the kernel shape
  int split_rows;  // rows of one split partial: 32 * waves of the kernel shape (32, 64, 128)
  int num_wg;      // persistent workgroups
  int max_splits;  // num_wg + n_units
  // Sparse bf16 decode by head group: 32-row groups per sequence unit, index
  // ranges per group (one workgroup each) and index entries per wave.
  int hg_groups, hg_splits, hg_span;
};

// The head-group sparse decode splits an item's index list over at most this
// many workgroups, and only when there are fewer items than this bound.
constexpr int kMaxHgSplits = 8;
constexpr int kMaxHgSplitItems = 4096;

struct WsLayout {
  size_t work;   // int32 [(num_wg + 1) * 2]   (first unit, first tile) per WG
  size_t cost;   // int32 [n_units + 1]        prefix of per-unit cost
  size_t meta;   // int32 [n_units * 4]        n_tiles, split_base, n_splits, g_first
  size_t plse;   // f32   [max_splits * split_rows]   partial log2-sum-exp
  size_t psc;    // f32   [max_splits * split_rows]   partial row scale (largest |O/l|)
  size_t po;     // f16   [max_splits * split_rows * 512] partial O/l divided by the row scale
                 // (the head-group sparse kernel: f32 O/l, 32-row ranges)
  size_t total;
};

WsLayout ws_layout(const Geometry& g);

struct DecodeArgs {
  const uint16_t* q_nope;
  const uint16_t* q_rope;
  const uint8_t* kv;
  const float* kv_scales;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;
  uint16_t* out;
  float* lse;
  int32_t* ws_work;
  int32_t* ws_cost;
  int32_t* ws_meta;
  float* ws_plse;
  float* ws_psc;
  float* ws_po;
  int bt_stride;
  int num_pages;
  int B, Sq, H, topk;
  int n_su, m_full, row_blocks, n_units, num_wg, split_rows;
  int causal;
  float scale_log2;  // softmax_scale * log2(e)
  int hg_groups, hg_splits, hg_span;
  int fold_plan;  // the main pass computes its own schedule (no scheduling launch)
};

// Cache append: the Sq new latent rows of every sequence into their slots.
struct AppendArgs {
  const uint16_t* src;        // bf16 [B, Sq, 576]
  uint8_t* kv;                // [num_pages, 64, 576] bf16 or e4m3fn
  float* kv_scales;           // fp32 [num_pages, 64] (fp8 only)
  const int32_t* block_table; // [B, bt_stride]
  const int32_t* seqlens;     // [B], the new tokens included
  int B, Sq, bt_stride, num_pages;
};
hipError_t launch_append(const AppendArgs& a, bool fp8, hipStream_t stream);

// DSA block top-k selection from per-block indexer scores.
constexpr int kMaxSelect = 256;       // selected blocks per query
constexpr int kMaxSelBlocks = 16384;  // blocks per score row (keys in LDS)
struct SelectArgs {
  const float* scores;      // [B, Sq, nbk]
  const int32_t* seqlens;   // [B], the new tokens included
  int32_t* indices;         // [B, Sq, n_select * 64]
  int B, Sq, nbk, n_select, n_init, n_local;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

// Per-head projections around the absorbed decode: C[m, h, :] = A[m, h, :] Bt[h]^T.
constexpr int kDHead = 128;  // head dimension d_h
struct ProjArgs {
  const uint16_t* a;  // bf16 [M, H, K]
  const uint16_t* w;  // bf16 [H, N, K]
  uint16_t* c;        // bf16 [M, H, N]
  int M, H;
};
hipError_t launch_proj(const ProjArgs& a, bool absorb, hipStream_t stream);

// The absorbed decode layer (mla_layer.hip): the query absorption with the
// split-KV scheduling pass as one more workgroup of the same launch.
struct LayerArgs {
  DecodeArgs d;  // the decode (q_nope and out point into the workspace)
  ProjArgs pa;   // absorption: a = q_c, w = W_UK^T, c = q_nope, M = B*Sq
};
hipError_t launch_absorb_plan(const LayerArgs& la, hipStream_t stream);

// Non-absorbed prefill over decompressed per-head Q/K (192 dims) and V (128).
struct PrefillArgs {
  const uint16_t* q;  // bf16 [B, T, H, 192]
  const uint16_t* k;  // bf16 [B, T, H, 192]
  const uint16_t* v;  // bf16 [B, T, H, 128]
  uint16_t* out;      // bf16 [B, T, H, 128]
  float* lse;         // fp32 [B, T, H]
  int B, T, H, causal;
  float scale;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Stages of a decode call (bit mask).
constexpr int kStagePlan = 1, kStageAttend = 2, kStageCombine = 4, kStagesAll = 7;

// The decode behind mla_decode / mla_sparse_decode / mla_attend: validates
// everything on the host, then enqueues the selected stages with the given
// workspace.  Sets the calling thread's error string on failure.
mla_status run_decode(const void* q_nope, const void* q_rope, const void* kv_pages,
                      const float* kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                      const int32_t* block_table, int bt_stride, const int32_t* cache_seqlens,
                      const int32_t* indices, int topk, int B, int Sq, int H, float softmax_scale,
                      int causal, void* out, float* lse, void* workspace, size_t ws_bytes,
                      int num_wg, int planned, hipStream_t stream, int stages = kStagesAll);
// Records `msg` as the calling thread's error detail and returns s.
mla_status fail_status(mla_status s, const char* msg);

hipError_t launch_plan(const Geometry& g, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode(const Geometry& g, const DecodeArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_combine(const Geometry& g, const DecodeArgs& a, hipStream_t stream);
// Sparse decode of a bf16 cache by head group (mla_sparse.hip): the main
// kernel, and when index lists are split over workgroups the merge of their
// partials; no scheduling pass.
hipError_t launch_sparse_hg(const Geometry& g, const DecodeArgs& a, hipStream_t stream);
inline bool uses_hg(const Geometry& g, bool fp8) { return g.sparse && !fp8; }

}  // namespace mla
