/*
 * mla.h -- C ABI of the weight-absorbed MLA decode library (libmla.so, gfx950).
 *
 * What the library computes.  Multi-head Latent Attention caches, per token,
 * only a 512-dim joint latent c^KV plus a 64-dim decoupled RoPE key k^R
 * ("MLA & DSA 推理性能优化指南" §1.1 figure; §5.1 table: d_c = 512,
 * d_rope = 64).  At decode time W_UK is absorbed into the query, so each head
 * scores the cached latent directly ("MLA 在极长上下文下的显存带宽突围",
 * section "运行期矩阵吸收避免潜在张量展开"):
 *
 *     z_j  = softmax_scale * ( q_nope . c_j  +  q_rope . k_rope_j )
 *     out  = sum_j softmax(z)_j * c_j          (512 dims per head)
 *     lse  = ln sum_j exp(z_j)                 (natural log)
 *
 * The same latent rows serve as keys (all 576 dims) and values (the first
 * 512), so every head of a sequence reads the same 1152 bytes per cached
 * token ("MLA & DSA 推理性能优化指南" §4.1).  The sparse variant attends only
 * over a given list of token positions, the DSA top-k selection of
 * "MLA & DSA 推理性能优化指南" §1.2 and §4.2.
 *
 * Data layout (all tensors dense, row-major, no strides):
 *   q_nope        bf16  [B, Sq, H, 512]
 *   q_rope        bf16  [B, Sq, H, 64]
 *   kv_pages      [num_pages, 64, 576]: per token the row [c (0..511) | k_rope
 *                 (512..575)]; bf16, or one OCP e4m3fn byte per element
 *   kv_scales     fp32  [num_pages, 64]: per-token dequant scale (fp8 only);
 *                 a token's value is e4m3fn(code) * scale
 *   block_table   int32 [B, bt_stride]: physical page of each 64-token logical
 *                 page of sequence b
 *   cache_seqlens int32 [B]: tokens in the cache of sequence b, the Sq new
 *                 tokens included
 *   indices       int32 [B, Sq, topk]: logical token positions (sparse only)
 *   out           bf16  [B, Sq, H, 512]
 *   lse           fp32  [B, Sq, H]
 *
 * Visibility.  Dense: token j of sequence b is visible to query s iff
 * j < L_b and, when causal != 0, j <= L_b - Sq + s.  Sparse: the listed
 * positions with 0 <= idx < L_b (no causal rule; entries are expected to be
 * distinct).  In both, a token whose logical page p has p >= bt_stride or a
 * block_table entry outside [0, num_pages) is not visible.  Cache bytes of
 * tokens that are not visible never influence results (they may hold NaN).
 * A query with no visible token gets out = 0 and lse = -inf.
 *
 * Ownership and execution.  Every pointer except those documented as host
 * pointers is a device pointer owned by the caller.  Calls validate their
 * arguments on the host, then only enqueue kernels on `stream`: they never
 * allocate or free device memory and never synchronise, so they can be
 * captured into a HIP graph.  The only library state is a per-device cache
 * of the compute-unit count and a thread-local error string.
 *
 * Errors.  Every entry point returns an mla_status.  All validation happens
 * before anything is enqueued, so a call that returns a validation error has
 * not touched `out`, `lse` or the workspace.  MLA_ERR_HIP means a launch
 * failed; `out`/`lse` are then undefined.  mla_last_error() gives a detail
 * string for the calling thread's last failing call.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_DC = 512,   /* latent (value) dims, d_c */
  MLA_DROPE = 64, /* decoupled RoPE key dims, d_rope */
  MLA_DLAT = 576, /* cached dims per token, d_c + d_rope */
  MLA_PAGE = 64,  /* tokens per cache page */
  MLA_MAX_ROWS_PER_UNIT = 128
};

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* a size or scalar argument is out of range */
  MLA_ERR_UNSUPPORTED = 3, /* valid request this build does not handle */
  MLA_ERR_ALIGN = 4,       /* a pointer breaks the alignment rule below */
  MLA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  MLA_ERR_HIP = 6          /* a HIP call or kernel launch failed */
} mla_status;

typedef enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3 = 1 } mla_kv_dtype;

/*
 * Bytes of device workspace a call with these sizes needs (0 on invalid
 * sizes).  topk = 0 selects the dense path, topk > 0 the sparse path.
 * num_wg is the number of persistent workgroups the work is spread over;
 * 0 means one per compute unit of the current device, or four per compute
 * unit when a scheduling unit has at most 32 query rows (Sq*H <= 32 dense,
 * H <= 32 sparse), whose one-wave workgroups share a unit.  The same
 * (B, Sq, H, topk, num_wg) must be passed to mla_plan / mla_decode /
 * mla_sparse_decode with a workspace of at least this size.  The size does
 * not depend on the cache lengths.
 */
size_t mla_workspace_size(int B, int Sq, int H, int topk, int num_wg);

/*
 * Split-KV scheduling pass: reads cache_seqlens on the device and writes the
 * work partition (which workgroup processes which 32-token chunks of which
 * sequence, and where each partial result goes) into the workspace.  It is
 * what mla_decode / mla_sparse_decode run first when `planned` is 0.  Run it
 * once per decode step and pass planned = 1 to every layer's call to reuse
 * the partition (valid while cache_seqlens and the sizes stay the same).
 * Alignment: workspace 256 B.
 */
mla_status mla_plan(const int32_t *cache_seqlens, int B, int Sq, int H, int topk, int num_wg,
                    void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Dense absorbed MLA decode (see the definition above).
 *   kv_dtype      MLA_KV_BF16, or MLA_KV_FP8_E4M3 with kv_scales non-NULL
 *   num_pages     pages in kv_pages (>= 1)
 *   bt_stride     int32 entries per block_table row (>= 1)
 *   softmax_scale finite positive multiplier of the scores (e.g. 1/sqrt(192))
 *   causal        nonzero: query s sees tokens j <= L_b - Sq + s
 *   planned       nonzero: mla_plan already filled this workspace
 * Limits: 1 <= Sq*H; sequences with Sq*H > 128 rows are processed as
 * several 128-row blocks, each reading the cache once.  The schedule counts
 * work in 32-bit units of 32 tokens: each row block's sequence is cut to
 * (2^31 - 2^17) / (row blocks of the whole decode) - 8 chunks of 32 tokens
 * (past 6e10 tokens in all, far beyond any cache that fits in memory).
 * Alignment: q_nope, q_rope, kv_pages, kv_scales, out 16 B; workspace 256 B.
 */
mla_status mla_decode(const void *q_nope, const void *q_rope, const void *kv_pages,
                      const float *kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                      const int32_t *block_table, int bt_stride, const int32_t *cache_seqlens,
                      int B, int Sq, int H, float softmax_scale, int causal, void *out,
                      float *lse, void *workspace, size_t ws_bytes, int num_wg, int planned,
                      hipStream_t stream);

/*
 * mla_decode without a caller-supplied workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split workspace is a static device
 * array inside the library, MLA_NOALLOC_SCRATCH_BYTES (96 MiB) per device,
 * which the library holds on every device it runs on until the process
 * ends.  Arguments and results are those of mla_decode (which always plans:
 * there is no `planned`); nothing is allocated or freed.  A request whose
 * workspace (mla_workspace_size with topk = 0) exceeds the array returns
 * MLA_ERR_WORKSPACE before anything is enqueued; the dense named workloads
 * fit on a 256-CU device with num_wg = 0.  Every call on one device shares
 * that device's array: calls whose executions overlap on one device (on
 * different streams, or from different threads) race and give undefined
 * results; calls ordered on one stream are safe.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)
mla_status mla_decode_noalloc(const void *q_nope, const void *q_rope, const void *kv_pages,
                              const float *kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                              const int32_t *block_table, int bt_stride,
                              const int32_t *cache_seqlens, int B, int Sq, int H,
                              float softmax_scale, int causal, void *out, float *lse, int num_wg,
                              hipStream_t stream);

/*
 * Sparse (DSA top-k) absorbed MLA decode: query (b, s) attends over the
 * positions indices[b, s, 0..topk) (see "Visibility" above).  Arguments as
 * mla_decode, plus indices and topk (>= 1); there is no causal rule.  Each
 * (b, s) is scheduled as its own unit of H rows.
 */
mla_status mla_sparse_decode(const void *q_nope, const void *q_rope, const void *kv_pages,
                             const float *kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                             const int32_t *block_table, int bt_stride,
                             const int32_t *cache_seqlens, const int32_t *indices, int topk,
                             int B, int Sq, int H, float softmax_scale, void *out, float *lse,
                             void *workspace, size_t ws_bytes, int num_wg, int planned,
                             hipStream_t stream);

/*
 * The three stages that mla_decode / mla_sparse_decode run, for callers that
 * schedule them separately (e.g. to time or overlap them):
 *   mla_plan     split-KV partition (above)
 *   mla_attend   the main pass: streams every 32-token chunk of every
 *                sequence once from HBM and computes softmax attention over
 *                it for all query rows of that sequence; writes out/lse of
 *                sequences that one workgroup finished alone, and partial
 *                results (normalised output and log-sum-exp per row and
 *                split) into the workspace for the others
 *   mla_combine  merges those partials by log-sum-exp into out/lse, and
 *                writes out = 0, lse = -inf for rows that see no token
 * mla_attend requires a workspace that mla_plan filled for the same sizes;
 * mla_combine requires the mla_attend that wrote the partials.  indices ==
 * NULL with topk == 0 selects the dense path (then causal applies); the
 * other arguments mean what they mean for mla_decode / mla_sparse_decode.
 */
mla_status mla_attend(const void *q_nope, const void *q_rope, const void *kv_pages,
                      const float *kv_scales, mla_kv_dtype kv_dtype, int num_pages,
                      const int32_t *block_table, int bt_stride, const int32_t *cache_seqlens,
                      const int32_t *indices, int topk, int B, int Sq, int H,
                      float softmax_scale, int causal, void *out, float *lse, void *workspace,
                      size_t ws_bytes, int num_wg, hipStream_t stream);

mla_status mla_combine(const int32_t *cache_seqlens, int B, int Sq, int H, int topk, void *out,
                       float *lse, void *workspace, size_t ws_bytes, int num_wg,
                       hipStream_t stream);

/*
 * Cache append of a decode step: writes the Sq new latent rows of every
 * sequence into their cache slots, the step that precedes attention
 * ("MLA & DSA 推理性能优化指南" §4, decode-flow figure: the output token is
 * appended to the cache).  Row s of sequence b, new_kv[b, s, :] (bf16
 * [B, Sq, 576], [c | k_rope]), goes to logical position j = L_b - Sq + s,
 * i.e. to kv_pages[block_table[b, j / 64], j % 64, :], where
 * L_b = cache_seqlens[b] already counts the new tokens (the convention of
 * mla_decode).  Rows with j < 0, with j / 64 >= bt_stride or with a page entry
 * outside [0, num_pages) are skipped.
 *   bf16 cache: the row is copied bit for bit.
 *   fp8 cache:  scale = max|x| / 448 over the row's 576 values (1 when all
 *               are zero); code = e4m3fn round-to-nearest-even of x / scale
 *               after clamping to +-448, computed in fp32 (correctly rounded
 *               division); the scale goes to kv_scales[page, j % 64].  Rows
 *               holding non-finite values get unspecified codes.
 * Distinct (b, s) must map to distinct slots (the caller's page allocation);
 * nothing else in the cache is written.
 * Alignment: new_kv, kv_pages 16 B; kv_scales, block_table, cache_seqlens 4 B.
 */
mla_status mla_kv_append(const void *new_kv, void *kv_pages, float *kv_scales,
                         mla_kv_dtype kv_dtype, int num_pages, const int32_t *block_table,
                         int bt_stride, const int32_t *cache_seqlens, int B, int Sq,
                         hipStream_t stream);

/*
 * DSA block top-k selection: the token lists mla_sparse_decode consumes,
 * from one indexer score per 64-token block ("MLA & DSA 推理性能优化指南"
 * §1.2 figure: Lightning Indexer scores, GPU top-k selection, block-aligned
 * k << L tokens; §6.1 table: 64-token blocks, 16 per query, 1 initial and
 * 2 local blocks always selected).  The indexer itself is not part of this.
 *   block_scores  fp32 [B, Sq, nbk]: score of block k (tokens 64k..64k+63)
 *                 for query (b, s); NaN counts as -inf
 *   cache_seqlens int32 [B], the Sq new tokens included
 *   indices       int32 [B, Sq, n_select * 64] (written)
 * Query s of sequence b sees L_s = L_b - Sq + s + 1 tokens (causal within
 * the step), i.e. nb = min(ceil(L_s / 64), nbk) blocks.  If nb <= n_select
 * every block is selected; otherwise blocks [0, n_init) and
 * [nb - n_local, nb) are, plus the n_select - n_init - n_local blocks between
 * them with the highest scores (ties: the lower block first).  The row lists
 * the selected blocks' 64 token positions each, blocks in ascending order,
 * with -1 for positions >= L_s and for unused slots.
 * Limits: 1 <= nbk <= 16384; 1 <= n_select <= 256; n_init, n_local >= 0 with
 * n_init + n_local <= n_select.  Alignment: 4 B.
 */
mla_status mla_dsa_select(const float *block_scores, int nbk, const int32_t *cache_seqlens, int B,
                          int Sq, int n_select, int n_init, int n_local, int32_t *indices,
                          hipStream_t stream);

/*
 * Per-head projections on either side of the absorbed decode.  With W_UK
 * absorbed into the query ("MLA 在极长上下文下的显存带宽突围", section on
 * absorbing the matrices at run time: q~ = q^C W^UK) the decode works in the
 * 512-dim latent space; W_UV brings its output back to the head dimension
 * ("MLA & DSA 推理性能优化指南" §1.1 figure: W_UK, W_UV map d_c to
 * d_h x n_h; §5.1: d_c = 512, d_h = 128).  M = B*Sq query rows, H heads.
 *
 * mla_absorb_query:  q_nope[m, h, n] = sum_k q_c[m, h, k] * w_uk_t[h, n, k]
 *   q_c     bf16 [M, H, 128]  per-head query (no RoPE part)
 *   w_uk_t  bf16 [H, 512, 128] W_UK stored transposed (w_uk_t[h, n, k] is
 *           W_UK[h][k][n], the weight that maps latent dim n to head dim k)
 *   q_nope  bf16 [M, H, 512]  written (fp32 accumulation, rounded to nearest)
 * mla_project_out:   o[m, h, j] = sum_d w_uv[h, j, d] * out_latent[m, h, d]
 *   out_latent bf16 [M, H, 512] (the decode's out)
 *   w_uv    bf16 [H, 128, 512]
 *   o       bf16 [M, H, 128]  written (fp32 accumulation, rounded to nearest)
 * Limits: M >= 1, 1 <= H <= 65535.  Alignment: 16 B.
 */
mla_status mla_absorb_query(const void *q_c, const void *w_uk_t, void *q_nope, int M, int H,
                            hipStream_t stream);
mla_status mla_project_out(const void *out_latent, const void *w_uv, void *o, int M, int H,
                           hipStream_t stream);

/*
 * The whole absorbed decode layer for a dense (non-sparse) cache ("MLA 最佳
 * 算子全景调研" §2: the gain of a fused decode comes from doing absorption,
 * attention and output projection together), in four launches: the query
 * absorption, the main pass (which schedules itself up to 2048 units;
 * beyond, the split-KV schedule runs as one more workgroup of the
 * absorption launch and the main pass reads it), the split merge and the
 * output projection.  Equivalent to
 * mla_absorb_query, then mla_decode on its q_nope, then mla_project_out on
 * the decode's out, with the same bf16 roundings of q_nope and of the
 * latent output between the steps.
 *   q_c, w_uk_t, w_uv, o  as mla_absorb_query / mla_project_out, with
 *                         M = B*Sq: q_c [B, Sq, H, 128], o [B, Sq, H, 128]
 *   q_rope, kv_pages, kv_scales, kv_dtype, num_pages, block_table,
 *   bt_stride, cache_seqlens, softmax_scale, causal, lse
 *                         as mla_decode (lse: natural-log lse of each row)
 *   workspace             >= mla_layer_workspace_size(B, Sq, H, num_wg)
 *                         bytes, 256-byte aligned; it also holds q_nope
 *                         and the merged 512-dim rows
 * Errors as mla_decode; nothing is enqueued on error.  Limits as mla_decode
 * and mla_absorb_query; B*Sq*H <= 2^22.
 */
size_t mla_layer_workspace_size(int B, int Sq, int H, int num_wg);
mla_status mla_decode_layer(const void *q_c, const void *w_uk_t, const void *q_rope,
                            const void *w_uv, const void *kv_pages, const float *kv_scales,
                            mla_kv_dtype kv_dtype, int num_pages, const int32_t *block_table,
                            int bt_stride, const int32_t *cache_seqlens, int B, int Sq, int H,
                            float softmax_scale, int causal, void *o, float *lse, void *workspace,
                            size_t ws_bytes, int num_wg, hipStream_t stream);

/*
 * Non-absorbed prefill: standard multi-head attention over K and V already
 * decompressed from the latent ("MLA & DSA 推理性能优化指南" §3.1: in
 * prefill c is decompressed into full K and V and a standard MHA kernel runs;
 * §5.1: 128 heads, d_h = 128, d_rope = 64).  Per head the query and key are
 * [nope (128) | rope (64)] and the value is 128 wide:
 *   out[b,t,h,:] = sum_j softmax_j(scale * q[b,t,h,:] . k[b,j,h,:]) v[b,j,h,:]
 *   lse[b,t,h]   = ln sum_j exp(scale * q[b,t,h,:] . k[b,j,h,:])   (natural log)
 * over j <= t when causal != 0, else over all j < T.
 *   q, k  bf16 [B, T, H, 192];  v bf16 [B, T, H, 128]
 *   out   bf16 [B, T, H, 128];  lse fp32 [B, T, H]   (written)
 * softmax_scale finite and > 0.  Limits: B, T >= 1; 1 <= H, B <= 65535;
 * B * T * H <= 2^31 / 192 and (T + 64) * H * 384 <= 2^32 (the kernel's byte
 * offsets within one sequence are 32-bit).  Alignment: q, k, v, out 16 B;
 * lse 4 B.
 */
mla_status mla_prefill(const void *q, const void *k, const void *v, int B, int T, int H,
                       float softmax_scale, int causal, void *out, float *lse, hipStream_t stream);

/* Static name of a status code ("MLA_OK", ...). */
const char *mla_status_str(mla_status s);

/* Detail message of the calling thread's last non-OK return ("" if none). */
const char *mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
