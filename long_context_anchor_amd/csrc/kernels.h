// Launch-side declarations of the libkascade kernels (host code).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kc {

constexpr int kMaxKvHeads = 64;

struct HeadMap {
  int32_t m[kMaxKvHeads];
};

// Split-K decode (dense anchor pass, or gathered reuse pass).
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sb, q_sh;            // query strides (elements)
  int64_t kv_sb, kv_sh, kv_sn;   // cache strides (elements)
  int32_t B, Hq, Hkv;
  int32_t n_keys;                // dense: N; gather: list length (topk)
  int32_t n_ctx;                 // keys in the cache (gather positions are clamped below it)
  float scale_log2;              // softmax scale * log2(e)
  int32_t keys_per_split, n_splits;
  float* scores;                 // [B,Hq,N] scaled log2-domain scores (anchor) or null
  float* part;                   // [B,Hq,n_splits,D+2]: m, l, o[D]
  const int32_t* idx;            // gather: anchor lists [B,Hkv_a,topk]
  int64_t idx_sb, idx_sg;
  HeadMap hm;
  uint32_t* hist0;               // [B*Hkv][2048] zeroed here for the pooling kernel, or null
  uint32_t* hist1;               // [B*Hkv][2048] zeroed here for the wide select, or null
  // paged caches: key j of batch b is row (j & (bs-1)) of physical block
  // table[b * table_stride + (j >> blk_shift)]; physical row number
  // R = block * blk_rows + row, address = base + g*kv_sh + R*kv_sn (elements)
  const int32_t* table;
  int32_t table_stride, blk_shift, num_blocks;
  int64_t blk_rows;
};

struct CombineArgs {
  const float* part;
  int32_t n_splits, BH;
  void* out;                     // [B*Hq, D] input dtype
  float* lse2;                   // [B*Hq] log2-domain lse (workspace), may be null
  float* lse_out;                // [B*Hq] natural-log lse, may be null
};

// Pooling of the anchor pass, fused with its split merge: workgroups
// x < ceil(N/1024) pool 1024 keys each (their group's lse comes from the
// splits' (m, l)); the G workgroups after them merge the splits of one query
// head each into out and lse_out.
struct PoolDecodeArgs {
  const float* scores;           // [B,Hq,N]
  const float* part;             // [B*Hq, n_splits, D+2] split partials (m, l, o), log2 domain
  int32_t n_splits;
  float* pooled;                 // [B,Hkv,N]
  uint32_t* hist0;               // [B*Hkv][2048]: counts of key bits 31..21 of pooled
  void* out;                     // [B*Hq, D] input dtype
  float* lse_out;                // [B*Hq] natural-log lse, may be null
  int32_t B, Hq, Hkv, N;
};

// Exact Top-k over rows.  mode 0: fixed n, k per row.  mode 1: prefill tile
// rows enumerated (b, t, g) with n = P_t, k = k_t from the rule.
struct SelectArgs {
  const float* src;
  int64_t row_stride;            // mode 0
  int32_t rows;
  int32_t n, k;                  // mode 0
  int32_t* idx;
  int64_t idx_stride;            // mode 0: row stride; mode 1: k_max
  int32_t mode;
  int32_t T, Hkv, N, tile, pct, round_to, k_min;   // mode 1
  int64_t packed_per_batch;      // mode 1: elements of one batch's packed rows
  int32_t cache_cap;             // rows up to this length are cached in LDS
  const uint32_t* hist0;         // [rows][2048] digit-0 histograms, or null
};

// Prefill kernels (bf16, d = 128, tile = 128).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sb, q_sh, q_sn;
  int64_t kv_sb, kv_sh, kv_sn;
  int32_t B, Hq, Hkv, N, T;
  float scale_log2;
  void* out;                     // [B,Hq,N,128] input dtype
  float* lse2;                   // [B,Hq,N] log2-domain lse (flash writes, pool reads)
  float* lse_out;                // [B,Hq,N] natural log, may be null
  float* pooled;                 // packed pooled rows
  int64_t packed_per_batch;
  const int32_t* idx;            // sparse: anchor tile lists [B,T,Hkv,k_max]
  int32_t k_max;
  int32_t pct, round_to, k_min;  // tile k rule
  int32_t half;                  // 1: fp16 q, k, v and out; 0: bf16
  HeadMap hm;
  // paged K/V (sparse only; table == null: contiguous caches).  Logical
  // position j of batch b is row j % 2^blk_shift of physical block
  // table[b * table_stride + (j >> blk_shift)], whose first row is physical
  // row block * blk_rows (rows of kv_sn elements from the cache base).
  const int32_t* table;
  int32_t table_stride, blk_shift, num_blocks;
  uint32_t blk_rows;
};

// Launchers: return hipSuccess or the launch error.
// Largest split of a gathered list (its indices are staged in LDS), and the
// split size the planner aims to stay under (the occupancy query assumes it).
constexpr int kMaxGatherKeys = 16384;
constexpr int kPlanMaxKeys = 4096;

// A 16-bit anchor split keeps its scores in LDS until it ends: over a paged
// cache at most kSpillMaxLds bytes of them, i.e. spill_max_keys(G, true)
// keys per split.
constexpr size_t kSpillMaxLds = 66 * 1024 + 1024;
// Over a contiguous cache a spilling workgroup runs alone on its CU (the
// floor below), so its score buffer may take most of the CU's LDS: up to
// kSpillMaxLdsOne bytes, i.e. 8192 keys per split for groups of up to 4
// (4336 for 8).  A paged split also stages its row list and keeps the
// smaller kSpillMaxLds.
constexpr size_t kSpillMaxLdsOne = 136 * 1024;
constexpr int kSpillMaxKeysOne = 8192;
// A 16-bit spilling workgroup asks for at least kSpillMinLds bytes of
// dynamic LDS: with its static LDS that is more than half of a CU's 160 KiB,
// so one spilling workgroup runs per CU (the planner's slot count sees it).
// Measured against two per CU: 131072 keys x 4 batches 407 -> 386 us per
// anchor layer, 32768 x 1 49.7 -> 49.2 us, identical results.
constexpr size_t kSpillMinLds = 80 * 1024;
// The dense (no spill, no list) pass takes the same floor when its splits
// are long (at least kDenseOneWgKeys keys, i.e. many rows of long context):
// 131072 keys x 4 batches 334 -> 316 us; at 32768 x 1 (short splits) one
// workgroup per CU was slower, so short splits keep two or more.
constexpr int kDenseOneWgKeys = 4096;
size_t spill_lds_bytes(int G, int keys_per_split);
int spill_max_keys(int G, bool paged);
hipError_t decode_set_max_lds();
// Split-K kernel variant: workgroups per CU without dynamic LDS, its static
// LDS, and the dynamic LDS of a split of kps keys.
hipError_t decode_splitk_attrs(int dtype, int G, bool gather, bool spill, bool paged, int* blocks,
                               size_t* static_lds);
size_t decode_splitk_dyn_lds(int dtype, int G, bool gather, bool spill, bool paged, int kps);
// paged: a.table is set (bf16 only)
hipError_t launch_decode_splitk(const DecodeArgs& a, int dtype, bool gather, hipStream_t s);
hipError_t launch_decode_combine(const CombineArgs& a, int dtype, hipStream_t s);
hipError_t launch_decode_pool(const PoolDecodeArgs& a, int dtype, hipStream_t s);
hipError_t launch_topk_select(const SelectArgs& a, hipStream_t s);

// Exact Top-k of a few long fp32 rows (decode pooled rows) by chunks of
// wide_chunk(n) keys over many workgroups, in three passes.  hist0 is
// complete (the pooling pass), hist1 is zero on entry.  Rows up to
// 96K keys use 1024-key chunks (twice the workgroups: 32K anchor layer 45.3
// -> 44.5 us, 66K-key rows 72.5 -> 71.7 us), longer rows 2048-key chunks
// (fewer chunk counts for the prefix of pass C: 128K x 4 anchor layer 383.8
// against 390.7 us with 1024).
constexpr int kWideChunk = 2048;
constexpr int kWideChunkShort = 1024;
constexpr int kWideShortMaxKeys = 98304;
inline int wide_chunk(int n) { return n <= kWideShortMaxKeys ? kWideChunkShort : kWideChunk; }
struct WideSelectArgs {
  const float* src;              // [rows][row_stride]
  int64_t row_stride;
  int32_t rows, n, k, chunks;
  int32_t* idx;                  // [rows][idx_stride]
  int64_t idx_stride;
  const uint32_t* hist0;         // [rows][2048]
  uint32_t* hist1;               // [rows][2048]
  uint32_t* cand;                // [rows][n] keys of the digit-0 bin, chunk c's at offset c*CH
  uint32_t* chunk_cnt;           // [rows][chunks][2] (keys above the digit-0 bin, candidates)
};
hipError_t launch_topk_select_wide(const WideSelectArgs& a, hipStream_t s);

// Fused anchor decode: one launch of co-resident workgroups (one per split
// of each (batch, KV head) row) runs the split-K pass with the scores kept
// in LDS, then, separated by three row-wide barriers, the lse and pooling,
// the digit-0 candidates and the exact threshold and index write.  Words the
// row's workgroups exchange are written and read with device-coherent
// accesses.
constexpr size_t kLdsPerCu = 160 * 1024;   // gfx950
constexpr int kFusedSyncWords = 64;    // per row: barrier count (word 0), departures (word 32)
struct FusedDecodeArgs {
  DecodeArgs d;                  // the anchor pass; d.part receives the splits' partials
  void* out;                     // [B,Hq,D] input dtype
  float* lse_out;                // [B,Hq] natural-log lse, or null
  int32_t* idx;                  // [B,Hkv,k] ascending
  float* pooled;                 // [B,Hkv,N] pooled probabilities, or null
  int32_t k;
  uint32_t* sync;                // [rows][kFusedSyncWords]: zero on entry, left zero
  uint32_t* status;              // bit 0 set when a row barrier gave up waiting
  uint32_t spin_limit;           // polls of a barrier before giving up
  uint32_t* hist0;               // [rows][2048]
  uint32_t* hist1;               // [rows][2048]
  uint32_t* cand;                // [rows][N] digit-0 candidates, split s's at offset s*kps
  uint32_t* cnt;                 // [rows][splits][2] (keys above the digit-0 bin, candidates)
  uint32_t cand_cap;             // candidates the LDS score buffer holds after the split's keys
};
hipError_t launch_anchor_fused(const FusedDecodeArgs& a, int dtype, hipStream_t s);
hipError_t anchor_fused_attrs(int dtype, int G, int kps, int* blocks, size_t* static_lds);
size_t anchor_fused_dyn_lds(int G, int kps);
size_t topk_select_lds_bytes(int cache_cap);
hipError_t topk_select_set_max_lds(size_t bytes);
hipError_t launch_prefill_flash(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_pool(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_sparse(const PrefillArgs& a, hipStream_t s);
size_t prefill_sparse_max_list();
size_t prefill_sparse_paged_max_list();
hipError_t prefill_set_max_lds();

// The per-tile k rule, identical on host and device.
__host__ __device__ inline int32_t tile_k_for_len(int32_t n, int32_t pct, int32_t round_to,
                                                  int32_t k_min) {
  int64_t r = round_to;
  int64_t tenth = r * (((int64_t)n * pct + 50 * r) / (100 * r));
  int64_t kk = tenth > k_min ? tenth : k_min;
  return (int32_t)(kk < n ? kk : n);
}

// Offset (elements) of packed pooled row (t, g) inside one batch.
__host__ __device__ inline int64_t packed_row_offset(int32_t t, int32_t g, int32_t Hkv,
                                                     int32_t tile, int32_t N) {
  // rows of tiles 0..t-1: Hkv * sum_{u<t} P_u ; P_u = min(N, tile*(u+1))
  int64_t full = (int64_t)(N / tile);   // tiles whose prefix is tile*(u+1)
  int64_t tt = t < full ? t : full;
  int64_t sum = (int64_t)tile * tt * (tt + 1) / 2 + (int64_t)(t - tt) * N;
  int64_t Pt = (int64_t)tile * (t + 1) < N ? (int64_t)tile * (t + 1) : N;
  return (int64_t)Hkv * sum + (int64_t)g * Pt;
}

// Calibration (calib.hip).
hipError_t launch_calib_sim(const float* pooled, const int32_t* idx, int L, int S, int Hkv, int N,
                            int k, float* sim, hipStream_t s);
hipError_t launch_layer_weight(const void* x, const void* y, int tokens, int dim, int dtype,
                               double* part, float* w, hipStream_t s);

}  // namespace kc
