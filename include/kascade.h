/*
 * kascade.h — C ABI of libkascade.so: Kascade cross-layer Top-k sparse
 * attention (anchor and reuse layers, decode and prefill) on MI355X (gfx950).
 *
 * The method is the one described on the pages about the paper "Kascade: A
 * Practical Sparse Attention Method for Long-Context LLM Inference"
 * (arXiv 2512.16391).  Citations name the page and its section:
 *   [Explainer] the 0h-n0.github.io page "論文解説: Kascade — レイヤー間スパーシティ
 *               再利用による実用的長文脈LLM推論高速化";
 *   [Abstract]  the paper's abstract (fugumt.com / montaan.com pages).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.   Every array argument is a DEVICE pointer, except `head_map`
 *             (a HOST array of n_kv_heads int32, validated on the host and
 *             passed to the kernels by value) and the shape/rule structs.
 * Ownership.  The caller allocates and frees every buffer, including the
 *             workspace (size from kascade_workspace_bytes).  The library
 *             never allocates device memory, never frees, and never
 *             synchronises (kascade_kernel_timer_read, a benchmark helper,
 *             is the one call that waits for recorded events).
 * Streams.    Work is enqueued asynchronously on `stream` (0 = null stream).
 * Layouts.    K and V caches are addressed through the element strides in
 *             kascade_shape (rows of d contiguous elements, 16-byte aligned;
 *             K and V share the strides): [B, Hkv, N_cap, d] and
 *             [B, N_cap, Hkv, d] both work.  Queries are [B, Hq, d] (decode) or [B, Hq, N, d]
 *             (prefill) through the q strides.  Outputs are CONTIGUOUS:
 *             out [B, Hq, d] / [B, Hq, N, d] in the input dtype, lse
 *             [B, Hq] / [B, Hq, N] fp32 (natural log).
 * GQA.        Query head h uses KV head h / (Hq / Hkv).
 * Scale.      shape.scale == 0 means 1/sqrt(head_dim).
 * Errors.     Every call returns KASCADE_OK (0) or a negative kascade_status.
 *             Arguments are validated before anything is launched: on a
 *             validation error nothing runs and no output is touched.  When a
 *             launch fails the call returns KASCADE_ERR_HIP, the outputs are
 *             undefined, and kascade_last_hip_error() (per thread) holds the
 *             hipError_t.
 * Determinism. No floating-point atomics: identical inputs give bitwise
 *             identical outputs.
 * Workspace.  Scratch only: no contents carry over between calls, any
 *             initial contents are fine.
 * Supported.  dtype F32 with head_dim 64, dtype BF16 or F16 with head_dim
 *             128 (one 256-byte K/V row in every case).  Prefill: BF16 or
 *             F16, head_dim 128, tile 128, batch 1..65535, Hq/Hkv in
 *             {1,2,4,8}, kv_stride_n * element size at most 32 MiB (64 rows
 *             span under 2 GiB).  Decode: ctx_len * kv_stride_n * element size below
 *             4 GiB (one head's rows; 16.7M keys at 256 bytes per row); a
 *             16-bit anchor decode also needs ctx_len <= 2048 * spill split (about
 *             8.6M keys for Hq/Hkv <= 4, 4.3M for 8), else KASCADE_ERR_SHAPE.
 * Threads.    Calls are thread-safe on distinct streams with distinct
 *             workspaces.
 */
#ifndef KASCADE_H
#define KASCADE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KASCADE_OK = 0,
  KASCADE_ERR_NULL = -1,       /* a required pointer is NULL                 */
  KASCADE_ERR_SHAPE = -2,      /* sizes/strides inconsistent or unsupported  */
  KASCADE_ERR_DTYPE = -3,      /* dtype x head_dim combination unsupported   */
  KASCADE_ERR_TOPK = -4,       /* topk outside [1, ctx_len] or bad rule      */
  KASCADE_ERR_HEADMAP = -5,    /* head_map entry outside [0, n_kv_heads)     */
  KASCADE_ERR_WORKSPACE = -6,  /* workspace smaller than required            */
  KASCADE_ERR_HIP = -7,        /* a HIP call failed (see last_hip_error)     */
  KASCADE_ERR_ARG = -8         /* another argument is out of range           */
} kascade_status;

typedef enum { KASCADE_F32 = 0, KASCADE_BF16 = 1, KASCADE_F16 = 2 } kascade_dtype;

typedef struct kascade_shape {
  int32_t batch;        /* B                                                */
  int32_t n_q_heads;    /* Hq                                               */
  int32_t n_kv_heads;   /* Hkv, divides Hq                                  */
  int32_t head_dim;     /* d                                                */
  int32_t ctx_len;      /* N: keys in the cache (decode) / prompt length    */
  int32_t dtype;        /* kascade_dtype of q, k, v and out                 */
  float scale;          /* softmax scale, 0 => 1/sqrt(d)                    */
  int32_t reserved;     /* must be 0                                        */
  int64_t q_stride_b, q_stride_h, q_stride_n;     /* in elements            */
  int64_t kv_stride_b, kv_stride_h, kv_stride_n;  /* in elements            */
} kascade_shape;

/* Prefill per-tile k rule ([Explainer] "Top-k設定", eq. k, with the query tile
 * of section "実装のポイント"): for tile t the causal prefix is
 * P_t = min(N, tile*(t+1)) and
 *   k_t = min(P_t, max(k_min, round_to * floor((P_t*pct + 50*round_to) /
 *                                               (100*round_to)))),
 * i.e. pct% of P_t rounded to the nearest multiple of round_to.  The
 * 32K-prompt workload uses {tile 128, pct 10, round_to 64, k_min 256}. */
typedef struct kascade_topk_rule {
  int32_t tile, pct, round_to, k_min;
} kascade_topk_rule;

/* ---- the four entry points ------------------------------------------- */

/* Anchor-layer decode.  [Explainer] "アンカーレイヤーと再利用レイヤー": an anchor
 * computes full attention and the Top-k key indices of its post-softmax
 * distribution; [Abstract]: the selection is exact and head-aware.
 *   out      [B,Hq,d]   dense attention output (input dtype)
 *   lse_out  [B,Hq]     fp32 logsumexp of the scaled scores, may be NULL
 *   topk_idx [B,Hkv,topk] int32: for each KV head g, the topk positions j
 *            with the largest pooled probability sum_{h in group g} P[b,h,j]
 *            (ties to the lower j), in ascending order
 *   pooled_out [B,Hkv,N] fp32 pooled probabilities, may be NULL
 * Requires 1 <= topk <= N. */
int kascade_anchor_decode(const kascade_shape* shape, const void* q, const void* k,
                          const void* v, int32_t topk, void* out, float* lse_out,
                          int32_t* topk_idx, float* pooled_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Anchor-layer decode in ONE launch (the same outputs as
 * kascade_anchor_decode; [Explainer] "アンカーレイヤーと再利用レイヤー": full
 * attention, then the exact Top-k of the pooled post-softmax probabilities).
 * The split-K workgroups keep their scores in LDS and run the pooling and the
 * exact selection themselves, separated by row-wide barriers, instead of the
 * four launches of kascade_anchor_decode.  With the same split plan as
 * kascade_anchor_decode the outputs are bitwise identical to it.
 *   Arguments as kascade_anchor_decode, plus
 *   max_polls  polls of each row barrier before the call gives up
 *              (0 = the default, 2^18: far above any normal wait).
 * Workspace (kascade_workspace_bytes op 6): unlike the other calls its first
 * 65792 bytes carry state, at the same offsets for every shape: bytes 0..3
 * are a status word and bytes 256..65791 row barrier counters, all of which
 * must be ZERO before the first call on a workspace (e.g. allocate it
 * zeroed); every call leaves the counters zero, so one workspace serves
 * calls of any shape it is large enough for.
 * A call whose barrier gave up sets status bit 0; its outputs are then
 * undefined (the caller reads the word after synchronising and clears it).
 * Requirements: BF16 or F16 (else KASCADE_ERR_DTYPE), not paged; all
 * workgroups of the launch must be resident on the GPU at once:
 * batch * n_kv_heads * splits <= CUs (one workgroup per CU; splits as in
 * kascade_anchor_decode, at most 256) and the split's scores must fit in LDS,
 * else KASCADE_ERR_SHAPE (the 32K and 64K single-sequence decodes of the
 * benchmark qualify, 128K x 4 does not).  Work running on the GPU at the
 * same time (other streams) delays the launch's workgroups, which is safe
 * while it ends within the barriers' wait (max_polls polls, about a second
 * by default).  Two fused calls must not run at the same time on one GPU
 * (calls on one stream are ordered and fine): each launch's resident
 * workgroups can hold the CUs the other's are waiting for, so both wait out
 * max_polls and report status bit 0 (nothing hangs, the outputs are
 * undefined). */
int kascade_anchor_decode_fused(const kascade_shape* shape, const void* q, const void* k,
                                const void* v, int32_t topk, void* out, float* lse_out,
                                int32_t* topk_idx, float* pooled_out, uint32_t max_polls,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Reuse-layer decode.  [Explainer] "アンカーレイヤーと再利用レイヤー" (attention
 * on the preceding anchor's selected keys only) and "ヘッドリマッピング" (each KV
 * head g of the reuse layer uses the list of anchor KV head head_map[g]).
 *   anchor_topk_idx [B,Hkv,topk] int32 device: the anchor's lists (any order,
 *            entries in [0,N); the caller guarantees this)
 *   head_map [Hkv] int32 HOST array, entries in [0,Hkv)
 *   out      [B,Hq,d]: for query head h, softmax over the listed keys of
 *            this layer's K (KV head h/G), renormalised over them, times V. */
int kascade_reuse_decode(const kascade_shape* shape, const void* q, const void* k,
                         const void* v, int32_t topk, const int32_t* anchor_topk_idx,
                         const int32_t* head_map, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Anchor-layer prefill (causal).  [Abstract]: tile-level operations in
 * prefill; [Explainer] "実装のポイント": 128-query tiles.
 *   out  [B,Hq,N,d] dense causal attention (input dtype); lse_out [B,Hq,N] or NULL
 *   tile_topk_idx [B,T,Hkv,k_max] int32, T = ceil(N/tile), k_max = k of the
 *        last tile: row (b,t,g) holds the k_t positions j < P_t with the
 *        largest pooled probability sum over the G heads of group g and the
 *        rows r of tile t of P[h,r,j] (P = 0 for j > r), ascending, ties to
 *        the lower j, then -1 up to k_max
 *   pooled_out: NULL or packed rows, row (b,t,g) at offset
 *        b*Hkv*S_T + Hkv*tile*t*(t+1)/2 + g*P_t (S_T = sum of all P_t), fp32 */
int kascade_anchor_prefill(const kascade_shape* shape, const void* q, const void* k,
                           const void* v, const kascade_topk_rule* rule, void* out,
                           float* lse_out, int32_t* tile_topk_idx, float* pooled_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Reuse-layer prefill (causal).  Row r of tile t, query head h attends to
 * J = { j in anchor_tile_topk_idx[b,t,head_map[h/G], 0:k_t] : j <= r } with a
 * softmax renormalised over J.  Lists must be ascending with -1 padding, as
 * written by kascade_anchor_prefill, and every J non-empty (true for the
 * rule's k_min >= tile).  head_map: HOST [Hkv]. */
int kascade_reuse_prefill(const kascade_shape* shape, const void* q, const void* k,
                          const void* v, const kascade_topk_rule* rule,
                          const int32_t* anchor_tile_topk_idx, const int32_t* head_map,
                          void* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Allocation-free reuse decode, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): kascade_reuse_decode without a workspace argument, same
 * kernels and the same results.  Its scratch (split partials [B*Hq, S, d+2]
 * then log2-lse [B*Hq], fp32, each part rounded up to 256 bytes; S = the
 * split count the library plans for topk keys, at most 2048) lives in a
 * static 8 MiB device array inside the library, one per GPU, held until the
 * process ends; the call allocates and frees nothing.  Calls whose scratch
 * would exceed 8 MiB return KASCADE_ERR_WORKSPACE before any launch (with
 * the default planning a call needs about B*Hq*min(topk/128, 512/(B*Hkv)+1)
 * * 520 bytes: 0.4 MB for 32 heads at k 3264, 1 MB for 4 x 32 heads at
 * k 13120).  Every call on a GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and give undefined results;
 * calls ordered on one stream are fine.  Nothing in the array needs to start
 * at zero.  Other arguments, errors and stream behaviour as for
 * kascade_reuse_decode. */
int kascade_reuse_decode_noalloc(const kascade_shape* shape, const void* q, const void* k,
                                 const void* v, int32_t topk, const int32_t* anchor_topk_idx,
                                 const int32_t* head_map, void* out, hipStream_t stream);

/* ---- paged KV caches (block tables) -------------------------------------- */

/* A paged K or V cache: key j of batch b lives in physical block
 * block_table[b * table_stride + j / block_size], row j % block_size; the
 * element (head g, row r, dim i) of physical block p is at
 *   cache + p * block_stride + g * shape->kv_stride_h + r * shape->kv_stride_n + i
 * (shape->kv_stride_b is not used).  Both caches share the layout and table.
 * block_size: a power of two; block_stride: a multiple of kv_stride_n, every
 * head's block_size rows inside it, num_blocks * (block_stride / kv_stride_n)
 * below 2^32.  Table entries and positions are clamped into range, so a bad
 * table cannot fault.  BF16 or F16 only. */
typedef struct kascade_paged_kv {
  const int32_t* block_table;   /* DEVICE int32 [B, table_stride], table_stride >= ceil(N / block_size) */
  int32_t table_stride;
  int32_t block_size;
  int32_t num_blocks;           /* physical blocks in each cache */
  int32_t reserved;             /* must be 0 */
  int64_t block_stride;         /* elements between physical blocks */
} kascade_paged_kv;

/* kascade_anchor_decode / kascade_reuse_decode over paged caches: the same
 * results for the same logical keys (positions in topk_idx and
 * anchor_topk_idx are logical).  Workspace sizes as for op 0 / op 1. */
int kascade_anchor_decode_paged(const kascade_shape* shape, const kascade_paged_kv* paged,
                                const void* q, const void* k_cache, const void* v_cache,
                                int32_t topk, void* out, float* lse_out, int32_t* topk_idx,
                                float* pooled_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
int kascade_reuse_decode_paged(const kascade_shape* shape, const kascade_paged_kv* paged,
                               const void* q, const void* k_cache, const void* v_cache,
                               int32_t topk, const int32_t* anchor_topk_idx,
                               const int32_t* head_map, void* out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* kascade_reuse_prefill over paged caches ([Explainer] "アンカーレイヤーと再利用
 * レイヤー" and "ヘッドリマッピング" as for the contiguous call): the same
 * results for the same logical keys.  shape->ctx_len is the prompt length N
 * (logical rows 0..N-1 of every batch, reached through the block table);
 * queries [B,Hq,N,d] through the q strides; positions in
 * anchor_tile_topk_idx are logical.  The tile's key list and its physical
 * rows are both staged in LDS, so k of the last tile is at most 12288
 * (prompts up to about 122K tokens at pct 10), else KASCADE_ERR_SHAPE.
 * No workspace is used (pass NULL, 0). */
int kascade_reuse_prefill_paged(const kascade_shape* shape, const kascade_paged_kv* paged,
                                const void* q, const void* k_cache, const void* v_cache,
                                const kascade_topk_rule* rule, const int32_t* anchor_tile_topk_idx,
                                const int32_t* head_map, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---- calibration (offline: choosing anchors and head maps) -------------- */

/* Per-KV-head similarity of every pair of layers a <= b over S calibration
 * queries: [Explainer] "レイヤー間類似度とアンカーレイヤー選択" (eq. sim) applied to
 * each pair of KV heads, the quantity "ヘッドリマッピング" maximises.
 *   pooled   [L, S, Hkv, n] fp32 device: each layer's pooled post-softmax rows
 *            (kascade_anchor_decode's pooled_out, one decode query per sample)
 *   topk_idx [L, S, Hkv, k] int32 device: the rows' Top-k positions
 *            (kascade_anchor_decode's topk_idx); entries are clamped into [0, n)
 *   sim      [L, L, Hkv, Hkv] fp32 device, out: for a <= b
 *            sim[a][b][ga][gb] = mean over s of
 *              sum_{j in topk_idx[a,s,ga]} pooled[b,s,gb,j] /
 *              sum_{j in topk_idx[b,s,gb]} pooled[b,s,gb,j];
 *            entries with a > b are not written.  fp64 sums, deterministic. */
int kascade_calib_head_similarity(int32_t L, int32_t S, int32_t n_kv_heads, int32_t n, int32_t k,
                                  const float* pooled, const int32_t* topk_idx, float* sim,
                                  hipStream_t stream);

/* Layer weight, [Explainer] eq. w: *w_out = 1 - mean over tokens t of
 * cos(x_t, y_t), x and y [tokens, dim] device arrays in `dtype` (F32,
 * BF16 or F16), the layer's input and output hidden states.  w_out: one float,
 * device.  NaN if some token has a zero vector.  Workspace: at least
 * kascade_layer_weight_workspace_bytes(tokens), contents irrelevant. */
int kascade_layer_weight(const void* x, const void* y, int32_t tokens, int32_t dim, int32_t dtype,
                         float* w_out, void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t kascade_layer_weight_workspace_bytes(int32_t tokens);

/* HOST.  Weighted similarity matrix for the anchor DP from a host copy of
 * kascade_calib_head_similarity's output: for a <= b
 *   S[a][b] = w[b] * mean over gb of max over ga of sim[a][b][ga][gb]
 * (each head of b at its best anchor head: the remapped similarity), 0 below
 * the diagonal.  w: HOST [L] or NULL (all 1).  S: HOST [L, L] doubles. */
int kascade_weighted_similarity(int32_t L, int32_t n_kv_heads, const float* sim, const float* w,
                                double* S);

/* HOST.  [Explainer] "動的計画法（Algorithm 1）": the M anchors (layer 0 among
 * them) maximising sum_l S[a(l)][l], a(l) the last anchor <= l; ties keep the
 * smallest start.  anchors: HOST [M] out, ascending; score: optional total. */
int kascade_select_anchors(int32_t L, int32_t M, const double* S, int32_t* anchors, double* score);

/* HOST.  [Explainer] "ヘッドリマッピング": head_maps [L, Hkv] out; for a layer b
 * reusing anchor a(b), head_maps[b][gb] = argmax over ga of
 * sim[a(b)][b][ga][gb] (ties to the lower ga); anchors get the identity.
 * anchors: HOST [M] ascending with anchors[0] == 0. */
int kascade_head_maps(int32_t L, int32_t n_kv_heads, const float* sim, const int32_t* anchors,
                      int32_t M, int32_t* head_maps);

/* ---- helpers ----------------------------------------------------------- */

/* op: 0 anchor_decode, 1 reuse_decode, 2 anchor_prefill, 3 reuse_prefill,
 * 4 dense_decode, 5 dense_prefill, 6 anchor_decode_fused.  Returns the
 * workspace bytes the op needs for this shape (0 if none), or 0 for an
 * invalid op/shape. */
size_t kascade_workspace_bytes(int op, const kascade_shape* shape, int32_t topk,
                               const kascade_topk_rule* rule);

/* k_t for a prefix of n keys under `rule` (same integer formula as the
 * kernels).  Returns -1 if the rule is invalid. */
int32_t kascade_topk_for_len(int32_t n, const kascade_topk_rule* rule);

/* Exact Top-k of fp32 rows: for each row r of `rows`, the k positions with
 * the largest scores[r*row_stride + j], j < n, ties to the lower j, written
 * ascending to idx[r*idx_stride + 0:k].  -0.0 equals +0.0; NaN rows give
 * unspecified indices.  No workspace. */
int kascade_topk_select_f32(const float* scores, int64_t row_stride, int32_t rows,
                            int32_t n, int32_t k, int32_t* idx, int64_t idx_stride,
                            hipStream_t stream);

/* Stream-read reference for measurement (not part of the method): reads the
 * `bytes` bytes at src (device, 16-byte aligned, bytes a positive multiple of
 * 16) once with the 16-byte nontemporal loads of the decode passes and sets
 * *sink ^= XOR of all its 32-bit words (sink: device, 4-byte aligned; the
 * caller zeroes it if it wants the plain XOR).  Asynchronous on `stream`;
 * KASCADE_ERR_NULL / KASCADE_ERR_ARG on bad arguments, nothing launched. */
int kascade_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Dense baselines with the same kernels and layouts: decode = anchor decode
 * without pooling/selection; prefill = the causal flash pass alone. */
int kascade_dense_decode(const kascade_shape* shape, const void* q, const void* k,
                         const void* v, void* out, float* lse_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
int kascade_dense_prefill(const kascade_shape* shape, const void* q, const void* k,
                          const void* v, void* out, float* lse_out, hipStream_t stream);

/* Per-kernel timing with HIP events recorded on the launching stream around
 * every launch of kernel `kernel_id` (ids below) while enabled.  enable()
 * resets the totals; read() waits for the recorded events (it is the only
 * call that waits) and returns the summed milliseconds and the launch
 * count.  Launch calls never wait: the event pool grows on the host as
 * needed.  Launches on a stream under graph capture are not timed.  Not
 * thread-safe (one timing thread at a time); meant for benchmarks. */
enum {
  KASCADE_K_DECODE_SPLITK = 0, KASCADE_K_DECODE_COMBINE = 1, KASCADE_K_DECODE_POOL = 2,
  KASCADE_K_TOPK_SELECT = 3, KASCADE_K_REUSE_DECODE = 4, KASCADE_K_PREFILL_FLASH = 5,
  KASCADE_K_PREFILL_POOL = 6, KASCADE_K_PREFILL_SPARSE = 7, KASCADE_K_ANCHOR_FUSED = 8,
  KASCADE_K_COUNT = 9
};
int kascade_kernel_timer_enable(int kernel_id, int enable);
int kascade_kernel_timer_read(int kernel_id, double* total_ms, int64_t* launches);

const char* kascade_status_str(int status);
int kascade_last_hip_error(void);
const char* kascade_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KASCADE_H */
