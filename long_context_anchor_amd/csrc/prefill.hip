// Prefill kernels (bf16 or fp16, head_dim 128, 128-query tiles) on gfx950 MFMA.
//
// Method: in prefill an anchor layer runs causal dense attention, pools the
// post-softmax probabilities of each 128-query tile over the tile's rows and
// the KV head's query group, and keeps the exact Top-k keys of every pooled
// tile row; a reuse layer runs causal attention over the anchor's list of
// its remapped KV head ([Abstract]: tile-level operations in prefill; page
// "論文解説: Kascade …", sections "アンカーレイヤーと再利用レイヤー",
// "ヘッドリマッピング" and "実装のポイント").
//
// Kernels
//   k_prefill_attn<false>  causal flash attention, writes O and the log2 lse
//   k_prefill_attn<true>   the same over a gathered key list (reuse layer)
//   k_prefill_pool<G>      recomputes S = Q K^T per (tile, KV head) and sums
//                          2^(S*c - lse2) over the G heads x 128 rows; the
//                          tile's queries stay in LDS, each wave owns whole
//                          64-key slices (no barrier in the key loop)
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, or _f16 for fp16 inputs; wave64).  Operand A is 32x16 with
// lane l holding row l%32, k = 8*(l/32)..+7; operand B is 16x32 with lane l
// holding column l%32, the same k; the 32x32 fp32 result gives lane l column
// l%32 and rows 8i + 4*(l/32) + j in register 4i+j.
//   attention: S^T = K Q^T (A = K rows from LDS, B = Q rows in registers),
//     so each lane owns one query and its softmax row statistics stay in
//     the lane (plus its partner lane l^32).  P^T in that C layout is
//     already the B operand of O^T = V^T P^T for a permuted key order of
//     each 16-key chunk; V stays [key][d] in LDS and its A operand is read
//     with the gfx950 transposing LDS load (ds_read_b64_tr_b16) in that
//     order.
//   pooling: S = Q K^T (A = Q fragments from LDS, B = K^T fragments held in
//     registers for a 64-key slice), so each lane owns one key column and
//     the pooled column sum is an in-lane sum.
#include "common.h"
#include "kernels.h"
#include "paged.h"

namespace kc {

namespace {

constexpr int kD = 128;
constexpr int kTileQ = 128;            // query rows per tile (4 waves x 32)
constexpr int kKB = 64;                // keys per block
constexpr int kKStride = kD + 8;       // bf16 per K row in LDS (272 B: conflict-free 16-byte reads)
constexpr int kVStride = kD + 32;      // bf16 per V row in LDS (320 B: conflict-free transposed reads)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool HALF>
KC_INLINE typename Fmt16<HALF>::v8 as_v8(const uint4& u) {
  u32x4 v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(typename Fmt16<HALF>::v8, v);
}
KC_INLINE uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
KC_INLINE void sts16(uint16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }


// Register staging of one block of 64 key rows between their global loads
// and their LDS store, so the loads of a later block are in flight while the
// current one is used.  A block is 64 rows x 16 chunks of 16 bytes; thread
// tid owns chunks tid + i*NT.  Per-thread row offsets are fixed, so a dense
// block needs only its (scalar) base address.
template <int NT, int STRIDE = kKStride>
struct RowStager {
  static constexpr int U = kKB * 16 / NT;
  uint4 k[U];

  KC_INLINE static int row(int i) { return (threadIdx.x + i * NT) >> 4; }
  KC_INLINE static int chunk(int i) { return (threadIdx.x + i * NT) & 15; }

  // Rows kb .. kb+63 of a dense cache.  Block rows >= nvalid load the last
  // valid row instead (real, finite cache data): their scores are masked to
  // -inf and their probabilities are 0, so nothing is zeroed here and the
  // loads stay in flight until the LDS store one step later.
  KC_INLINE void load_dense(const char* blk, int64_t row_bytes, int nvalid) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int rr = min(row(i), max(nvalid - 1, 0));
      k[i] = ld16(blk + (int32_t)(rr * (int32_t)row_bytes) + chunk(i) * 16);
    }
  }
  // Gathered rows pos[rr] (block-relative rows rr < nvalid); missing rows
  // (-1 or past the list) load cache row 0 and are masked the same way.
  // nvalid >= 1, so every list read is clamped into the block's entries and
  // issued unconditionally: the reads go out together and one wait covers
  // them (a read guarded by rr < nvalid becomes a branch and a wait per row).
  KC_INLINE void load_gather(const char* base, int64_t row_bytes, const int32_t* pos, int nvalid) {
    int p[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int rr = row(i);
      const int v = pos[min(rr, nvalid - 1)];
      p[i] = rr < nvalid ? v : -1;
    }
#pragma unroll
    for (int i = 0; i < U; ++i) k[i] = ld16(base + (int64_t)(p[i] < 0 ? 0 : p[i]) * row_bytes + chunk(i) * 16);
  }
  // Physical rows rows[rr] of a paged cache (block-relative rows rr <
  // nvalid); missing rows load physical row 0 and are masked the same way.
  KC_INLINE void load_rows(const char* base, int64_t row_bytes, const int32_t* rows, int nvalid) {
    uint32_t p[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int rr = row(i);
      const uint32_t v = (uint32_t)rows[min(rr, nvalid - 1)];
      p[i] = rr < nvalid ? v : 0u;
    }
#pragma unroll
    for (int i = 0; i < U; ++i) k[i] = ld16(base + (uint64_t)p[i] * (uint64_t)row_bytes + chunk(i) * 16);
  }
  // rows as [key][d] (padded rows of STRIDE bf16)
  KC_INLINE void store(uint16_t* sk) const {
#pragma unroll
    for (int i = 0; i < U; ++i) sts16(sk + row(i) * STRIDE + chunk(i) * 8, k[i]);
  }
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// V^T fragment (MFMA A operand, 32 d rows x 16 keys) read transposed from V
// stored as [key][d]: ds_read_b64_tr_b16 hands lane i of each 16-lane group
// element (i & 3) of the 8-byte row addressed by lane 4e + (i >> 2), as its
// element e.  Lane l (half h = l/32, group g16 = (l/16)&1, j = l&15)
// addresses keys kc + 4h + (j>>2) (and +8) at d = d0 + 16*g16 + 4*(j&3), so
// it receives d = d0 + l%32 for keys kc + 4h + {0..3, 8..11}: the order of
// the B operand P^T taken from the S^T accumulator layout.
template <bool HALF>
KC_INLINE typename Fmt16<HALF>::v8 v_frag(const uint16_t* sv, int kc, int d0, int lane) {
  const int h = lane >> 5, g16 = (lane >> 4) & 1, j = lane & 15;
  const uint16_t* p0 = sv + (kc + 4 * h + (j >> 2)) * kVStride + d0 + 16 * g16 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * kVStride));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(typename Fmt16<HALF>::v8, v);
}

// XCD-aware work order.  Workgroups are dispatched round-robin over the 8
// XCDs (each with its own L2), so launch id L runs on XCD L % 8.  Work items
// are ordered (batch, KV head, tile from the longest causal prefix down,
// query head of the group fastest) and each XCD takes one contiguous eighth:
// the query heads sharing a KV head and the tiles streaming the same keys
// run on the same L2.  Returns false for the padding ids of the last eighth.
constexpr int kXcds = 8;
KC_INLINE bool xcd_work_item(int total, int G, int T, int Hkv, int& t, int& h, int& b) {
  const int L = blockIdx.x;
  const int per = (total + kXcds - 1) / kXcds;
  const int w = (L % kXcds) * per + L / kXcds;
  if (w >= total) return false;
  const int hh = w % G;
  int rest = w / G;
  t = T - 1 - rest % T;
  rest /= T;
  const int g = rest % Hkv;
  b = rest / Hkv;
  h = g * G + hh;
  return true;
}
inline int xcd_grid(int total) { return (total + kXcds - 1) / kXcds * kXcds; }

// S^T = K_block Q^T for the wave's 32 queries: two 32-key tiles.
// The two key tiles are independent accumulation chains; alternating them
// keeps a dependent MFMA one issue away from its predecessor.
template <bool HALF>
KC_INLINE void qk_block(const uint16_t* sk, const typename Fmt16<HALF>::v8* qf, int l32, int hf,
                        f32x16_t* s) {
  s[0] = f32x16_t{};
  s[1] = f32x16_t{};
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const auto kf = as_v8<HALF>(lds16(sk + (kt * 32 + l32) * kKStride + ds * 16 + hf * 8));
      s[kt] = Fmt16<HALF>::mfma(kf, qf[ds], s[kt]);
    }
  }
}

// One workgroup = one (query tile, query head, batch); 4 waves x 32 rows.
// GATHER: the keys are the tile's list for KV head head_map[g] (ascending,
// staged in LDS once), masked per row by position <= row.
//
// Software pipeline over 64-key blocks j: while the MFMAs of S_{j+1} =
// K_{j+1} Q^T run, the VALU does the softmax of S_j, then O^T += V_j^T P_j^T.
// K is double-buffered in LDS (K_{j+1} is written one block ahead), V is
// single-buffered (V_j is written at the start of step j); global loads of
// K_{j+2} and V_{j+1} are in flight during step j.
template <bool GATHER, int WAVES, bool HALF, bool DB, bool PAGED = false>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void k_prefill_attn(const PrefillArgs a) {
  static_assert(GATHER || !PAGED, "paged caches are read through a key list");
  typedef Fmt16<HALF> F;   // bf16 or fp16 elements
  typedef typename F::v8 v8;
  constexpr int NT = 64 * WAVES;
  // DB: K and V double-buffered (one barrier per block); otherwise V is
  // single-buffered, which leaves more LDS for a long staged key list
  constexpr int NVB = DB ? 2 : 1;
  __shared__ __align__(16) uint16_t sk[2][kKB * kKStride];
  __shared__ __align__(16) uint16_t sv[NVB][kKB * kVStride];
  extern __shared__ int32_t slist[];
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int l32 = lane & 31, hf = lane >> 5;
  const int N = a.N;
  // Work item and this wave's (query head, 32-row slice):
  //   dense, 8 waves : 256 consecutive rows (two tiles) of one query head;
  //   gather, 8 waves: one tile of two query heads of the group (same list);
  //   4 waves        : one tile of one query head.
  int t, h, b, row0, kend;
  if (WAVES == 8 && !GATHER) {
    const int Tp = (a.T + 1) / 2;
    int pr;
    if (!xcd_work_item(Tp * a.Hq * a.B, G, Tp, a.Hkv, pr, h, b)) return;
    row0 = pr * 2 * kTileQ + wave * 32;
    t = pr * 2 + (wave >> 2);
    kend = min(N, 2 * kTileQ * (pr + 1));
  } else if (WAVES == 8) {
    int hp;
    if (!xcd_work_item(a.T * (a.Hq / 2) * a.B, G / 2, a.T, a.Hkv, t, hp, b)) return;
    h = 2 * hp + (wave >> 2);
    row0 = t * kTileQ + (wave & 3) * 32;
    kend = min(N, kTileQ * (t + 1));
  } else {
    if (!xcd_work_item(a.T * a.Hq * a.B, G, a.T, a.Hkv, t, h, b)) return;
    row0 = t * kTileQ + wave * 32;
    kend = min(N, kTileQ * (t + 1));
  }
  const int g = h / G;
  const int r = row0 + l32;
  const float c = a.scale_log2;

  // queries as the B operand: lane holds row r, d = 16*ds + 8*hf + 0..7
  v8 qf[8];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)min(r, N - 1) * a.q_sn) * 2;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const uint4 u = ld16(qp + (ds * 16 + hf * 8) * 2);
      qf[ds] = as_v8<HALF>(r < N ? u : make_uint4(0, 0, 0, 0));
    }
  }
  int nkeys = kend;
  // PAGED: the physical row of every listed key follows the list in LDS
  // (logical positions stay in slist for the causal mask)
  int32_t* const sphys = slist + a.k_max;
  if (GATHER) {
    nkeys = tile_k_for_len(kend, a.pct, a.round_to, a.k_min);
    const int32_t* list = a.idx + ((int64_t)(b * a.T + t) * a.Hkv + a.hm.m[g]) * a.k_max;
    for (int i = tid; i < nkeys; i += NT) {
      const int p = list[i];
      const int lp = (p >= 0 && p < N) ? p : -1;
      slist[i] = lp;
      if (PAGED) {
        // block clamped into the cache so a bad table cannot fault
        const uint32_t phys =
            lp >= 0 ? paged_row(a.table, a.table_stride, b, lp, N, a.blk_shift, a.num_blocks, a.blk_rows)
                    : 0u;
        sphys[i] = (int32_t)phys;
      }
    }
    __syncthreads();
  }
  const int64_t row_bytes = a.kv_sn * 2;
  // paged caches hold every batch's blocks: no batch offset
  const int64_t head_off = ((PAGED ? 0 : (int64_t)b * a.kv_sb) + (int64_t)g * a.kv_sh) * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.v) + head_off;
  const int nb = (nkeys + kKB - 1) / kKB;

  RowStager<NT> kr;
  RowStager<NT, kVStride> vr;
  // loads of block jb (K or V) into a stager
  auto load_blk = [&](RowStager<NT>& st, int jb) {
    const int kb = jb * kKB;
    if (PAGED) st.load_rows(kbase, row_bytes, sphys + kb, nkeys - kb);
    else if (GATHER) st.load_gather(kbase, row_bytes, slist + kb, nkeys - kb);
    else st.load_dense(kbase + (int64_t)kb * row_bytes, row_bytes, nkeys - kb);
  };
  auto load_vblk = [&](RowStager<NT, kVStride>& st, int jb) {
    const int kb = jb * kKB;
    if (PAGED) st.load_rows(vbase, row_bytes, sphys + kb, nkeys - kb);
    else if (GATHER) st.load_gather(vbase, row_bytes, slist + kb, nkeys - kb);
    else st.load_dense(vbase + (int64_t)kb * row_bytes, row_bytes, nkeys - kb);
  };

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  f32x16_t sA[2], sB[2];
  if constexpr (!DB) {
    load_blk(kr, 0);
    load_vblk(vr, 0);
    kr.store(sk[0]);
    if (nb > 1) load_blk(kr, 1);
    __syncthreads();
    qk_block<HALF>(sk[0], qf, l32, hf, sA);
  } else {
    // K_0, V_0 and K_1 in LDS; K_2 and V_1 in flight into the stagers
    load_blk(kr, 0);
    load_vblk(vr, 0);
    kr.store(sk[0]);
    vr.store(sv[0]);
    if (nb > 1) {
      load_blk(kr, 1);
      kr.store(sk[1]);
    }
    __syncthreads();
    qk_block<HALF>(sk[0], qf, l32, hf, sA);
    if (nb > 2) load_blk(kr, 2);
    if (nb > 1) load_vblk(vr, 1);
    __syncthreads();   // sk[0] is rewritten in step 0
  }

  // One pipeline step on block j: s_cur holds S_j; S_{j+1} goes to s_next.
  auto step = [&](int j, f32x16_t* s_cur, f32x16_t* s_next) {
    const int kb = j * kKB;
    if constexpr (!DB) {
      __syncthreads();   // every wave is done with V_{j-1} and K_j's LDS reads
      if (j + 1 < nb) kr.store(sk[(j + 1) & 1]);
      vr.store(sv[0]);
      __syncthreads();
      if (j + 2 < nb) load_blk(kr, j + 2);
      if (j + 1 < nb) load_vblk(vr, j + 1);
    } else {
      // Step j reads K_{j+1} and V_j, stored in step j-1; it stores K_{j+2}
      // over K_j and V_{j+1} over V_{j-1}, whose last readers finished
      // before the barrier that ended step j-1.
      if (j + 2 < nb) kr.store(sk[j & 1]);
      if (j + 1 < nb) vr.store(sv[(j + 1) & 1]);
      if (j + 3 < nb) load_blk(kr, j + 3);
      if (j + 2 < nb) load_vblk(vr, j + 2);
    }

    // causal mask inside the block (key position > query row) and empty slots
    // (a scalar, wave-uniform decision; the masked path is branch-free)
    bool need_mask;
    if (GATHER) {
      const int last = __builtin_amdgcn_readfirstlane(slist[min(nkeys, kb + kKB) - 1]);
      need_mask = (kb + kKB > nkeys) || (last > row0) || (last < 0);
    } else {
      need_mask = (kb + kKB - 1 > row0) || (kb + kKB > nkeys);
    }
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ri = 0; ri < 16; ++ri) {
          const int kk = kb + kt * 32 + 8 * (ri >> 2) + 4 * hf + (ri & 3);
          int p = GATHER ? slist[min(kk, nkeys - 1)] : kk;
          p = kk < nkeys ? p : -1;
          s_cur[kt][ri] = (p < 0 || p > r) ? kNegInf : s_cur[kt][ri];
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) mx = fmaxf(mx, s_cur[kt][ri]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescaling: the reference max m moves only when some row's block
    // max exceeds it by more than 2^8 (then every row of the wave updates
    // exactly), so p <= 2^8 and O, l stay well inside fp32 range.
    if (__any(mx * c > m + 8.f)) {
      const float mn = fmaxf(m, mx * c);
      const float alpha = mn == kNegInf ? 1.f : exp2f_fast(m - mn);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m = mn;
    }
    // a row whose max is still -inf has only masked scores in this block:
    // any finite reference gives them p = 2^-inf = 0
    const float mn = m == kNegInf ? 0.f : m;

    // One straight-line region: the MFMAs of S_{j+1} (issued unconditionally;
    // after the last block they read a stale buffer and are discarded), the
    // softmax of S_j, and O^T += V_j^T P_j^T, so the scheduler can interleave
    // VALU work with the matrix pipe.  Row sums stay fp32 on the unrounded P
    // (the log-sum-exp feeds the pooling pass).
    qk_block<HALF>(sk[(j + 1) & 1], qf, l32, hf, s_next);
    v8 pb[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kt = q4 >> 1, c2 = q4 & 1;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = exp2f_fast(fmaf(s_cur[kt][8 * c2 + e], c, -mn));
      l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      uint4 pk;
      pk.x = F::pack(p[0], p[1]);
      pk.y = F::pack(p[2], p[3]);
      pk.z = F::pack(p[4], p[5]);
      pk.w = F::pack(p[6], p[7]);
      pb[q4] = as_v8<HALF>(pk);
    }
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = F::mfma(v_frag<HALF>(sv[DB ? (j & 1) : 0], ch * 16, db * 32, lane), pb[ch], o[db]);
    }
    if constexpr (DB) __syncthreads();
  };
  for (int j = 0; j < nb; j += 2) {
    step(j, sA, sB);
    if (j + 1 < nb) step(j + 1, sB, sA);
  }

  // normalise and write: lane holds query r, d rows 32*db + 8i + 4*hf + j
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (r < N) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (((int64_t)b * a.Hq + h) * N + r) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = F::pack(o[db][4 * i + 0] * inv, o[db][4 * i + 1] * inv);
        w.y = F::pack(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * i + 4 * hf) = w;
      }
    }
    if (hf == 0) {
      const float lse2 = m + log2f_fast(lt);
      const int64_t li = ((int64_t)b * a.Hq + h) * N + r;
      if (a.lse2) a.lse2[li] = lse2;
      if (a.lse_out) a.lse_out[li] = lse2 * kLn2;
    }
  }
}

// Pooling with the tile's queries resident in LDS: one workgroup = one
// (query tile, KV head, batch) holds the 128 rows of HQ heads of the group
// (HQ*34 KiB) and the rows' -lse2/c; each wave owns whole 64-key slices of
// the causal prefix, keeps their K^T fragments in registers, and runs every
// held query row against them, so a key's pooled sum over the heads and
// rows stays in its lane and is written once.  No barrier inside the key
// loop: waves proceed independently.  Each Q fragment read from LDS feeds
// two MFMAs (the slice's two 32-key halves).
template <int G, bool HALF>
__global__ __launch_bounds__(1024) void k_prefill_pool(const PrefillArgs a) {
  typedef Fmt16<HALF> F;
  typedef typename F::v8 v8;
  constexpr int HQ = G < 4 ? G : 4;      // heads held per pass
  constexpr int PASSES = G / HQ;
  constexpr int NT = 1024, NW = NT / 64;
  extern __shared__ __align__(16) uint16_t dyn[];
  uint16_t* const sq = dyn;                                            // [HQ][128][kKStride]
  float* const nlse = reinterpret_cast<float*>(dyn + HQ * kTileQ * kKStride);   // [HQ][128]

  int t, g, b;
  if (!xcd_work_item(a.T * a.Hkv * a.B, 1, a.T, a.Hkv, t, g, b)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int N = a.N;
  const float c = a.scale_log2;
  const float inv_c = 1.0f / c;
  const int P = min(N, kTileQ * (t + 1));
  const int nsl = (P + kKB - 1) / kKB;
  const int64_t row_bytes = a.kv_sn * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * 2;
  float* prow = a.pooled + (int64_t)b * a.packed_per_batch + packed_row_offset(t, g, a.Hkv, kTileQ, N);

  for (int pass = 0; pass < PASSES; ++pass) {
    if (pass > 0) __syncthreads();   // every wave is done with the previous heads
    // queries of the pass's heads (rows past the prompt as zeros) and -lse2/c
    for (int i = tid; i < HQ * kTileQ * 16; i += NT) {
      const int ch = i & 15, rr = (i >> 4) % kTileQ, hq = i / (16 * kTileQ);
      const int h = g * G + pass * HQ + hq, r = t * kTileQ + rr;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (r < N)
        u = ld16(reinterpret_cast<const char*>(a.q) +
                 ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)r * a.q_sn) * 2 + ch * 16);
      sts16(sq + (hq * kTileQ + rr) * kKStride + ch * 8, u);
    }
    for (int i = tid; i < HQ * kTileQ; i += NT) {
      const int hq = i / kTileQ, rr = i % kTileQ, r = t * kTileQ + rr;
      const int h = g * G + pass * HQ + hq;
      nlse[i] = r < N ? -a.lse2[((int64_t)b * a.Hq + h) * N + r] * inv_c : 0.f;
    }
    __syncthreads();

    for (int sl = wave; sl < nsl; sl += NW) {
      const int kb = sl * kKB;
      // K^T fragments (MFMA B operand): lane holds key kb + 32*kt + l32 and
      // d = 16*ds + 8*hf .. +7; keys past the prefix load the last one (masked)
      v8 kf[2][8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = min(kb + kt * 32 + l32, P - 1);
        const char* kp = kbase + (int64_t)key * row_bytes + hf * 16;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) kf[kt][ds] = as_v8<HALF>(ld16(kp + ds * 32));
      }
      float cs0 = 0.f, cs1 = 0.f;
      const int j0 = kb + l32, j1 = kb + 32 + l32;
#pragma unroll 1
      for (int hq = 0; hq < HQ; ++hq) {
#pragma unroll 1
        for (int rs = 0; rs < 4; ++rs) {
          const int row0 = t * kTileQ + rs * 32;
          // every key after every row, or rows past the prompt: nothing to add
          if (kb > row0 + 31 || row0 >= N) continue;
          const float* nl = nlse + hq * kTileQ + rs * 32 + 4 * hf;
          f32x16_t acc0, acc1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 u = *reinterpret_cast<const float4*>(nl + 8 * i);
            acc0[4 * i + 0] = u.x; acc0[4 * i + 1] = u.y; acc0[4 * i + 2] = u.z; acc0[4 * i + 3] = u.w;
          }
          acc1 = acc0;
          const uint16_t* qrow = sq + (hq * kTileQ + rs * 32 + l32) * kKStride + hf * 8;
#pragma unroll
          for (int ds = 0; ds < 8; ++ds) {
            const v8 qa = as_v8<HALF>(lds16(qrow + ds * 16));
            acc0 = F::mfma(qa, kf[0][ds], acc0);
            acc1 = F::mfma(qa, kf[1][ds], acc1);
          }
          const bool need_mask = (kb + kKB - 1 > row0) || (kb + kKB > P) || (row0 + 32 > N);
          if (need_mask) {
#pragma unroll
            for (int ri = 0; ri < 16; ++ri) {
              const int rr = row0 + 8 * (ri >> 2) + 4 * hf + (ri & 3);
              const float p0 = exp2f_fast(acc0[ri] * c), p1 = exp2f_fast(acc1[ri] * c);
              cs0 += (j0 <= rr && rr < N && j0 < P) ? p0 : 0.f;
              cs1 += (j1 <= rr && rr < N && j1 < P) ? p1 : 0.f;
            }
          } else {
#pragma unroll
            for (int ri = 0; ri < 16; ++ri) {
              cs0 += exp2f_fast(acc0[ri] * c);
              cs1 += exp2f_fast(acc1[ri] * c);
            }
          }
        }
      }
      // the two half-waves hold complementary rows of the same keys
      cs0 += __shfl_xor(cs0, 32, 64);
      cs1 += __shfl_xor(cs1, 32, 64);
      const int j = hf ? j1 : j0;
      if (j < P) {
        const float v = hf ? cs1 : cs0;
        prow[j] = pass == 0 ? v : prow[j] + v;
      }
    }
  }
}

template <bool HALF>
hipError_t flash_h(const PrefillArgs& a, hipStream_t s) {
  const int Tp = (a.T + 1) / 2;
  hipLaunchKernelGGL((k_prefill_attn<false, 8, HALF, true>), dim3(xcd_grid(Tp * a.Hq * a.B)), dim3(512),
                     0, s, a);
  return hipGetLastError();
}

template <bool HALF, bool PAGED>
hipError_t sparse_h(const PrefillArgs& a, hipStream_t s) {
  // gathered variants keep V single-buffered: double buffering measured no
  // faster here and would take LDS from the staged list
  const size_t lds = (size_t)a.k_max * sizeof(int32_t) * (PAGED ? 2 : 1);
  if ((a.Hq / a.Hkv) % 2 == 0)
    hipLaunchKernelGGL((k_prefill_attn<true, 8, HALF, false, PAGED>), dim3(xcd_grid(a.T * (a.Hq / 2) * a.B)),
                       dim3(512), lds, s, a);
  else
    hipLaunchKernelGGL((k_prefill_attn<true, 4, HALF, false, PAGED>), dim3(xcd_grid(a.T * a.Hq * a.B)),
                       dim3(256), lds, s, a);
  return hipGetLastError();
}

// dynamic LDS of the pooling kernel: the held heads' 128 query rows and their -lse2/c
constexpr size_t pool_lds_bytes(int G) { return (size_t)(G < 4 ? G : 4) * kTileQ * (kKStride * 2 + 4); }

template <bool HALF>
hipError_t pool_h(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid(xcd_grid(a.T * a.Hkv * a.B)), block(1024);
  const int G = a.Hq / a.Hkv;
  const size_t lds = pool_lds_bytes(G);
  switch (G) {
    case 1: hipLaunchKernelGGL((k_prefill_pool<1, HALF>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_prefill_pool<2, HALF>), grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_prefill_pool<4, HALF>), grid, block, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_prefill_pool<8, HALF>), grid, block, lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool HALF>
hipError_t set_pool_lds_h() {
  const void* fs[] = {reinterpret_cast<const void*>(&k_prefill_pool<1, HALF>),
                      reinterpret_cast<const void*>(&k_prefill_pool<2, HALF>),
                      reinterpret_cast<const void*>(&k_prefill_pool<4, HALF>),
                      reinterpret_cast<const void*>(&k_prefill_pool<8, HALF>)};
  const int gs[] = {1, 2, 4, 8};
  for (int i = 0; i < 4; ++i) {
    const hipError_t e =
        hipFuncSetAttribute(fs[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)pool_lds_bytes(gs[i]));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool HALF, bool PAGED>
hipError_t set_lds_h(int bytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prefill_attn<true, 8, HALF, false, PAGED>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prefill_attn<true, 4, HALF, false, PAGED>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace

hipError_t launch_prefill_flash(const PrefillArgs& a, hipStream_t s) {
  return a.half ? flash_h<true>(a, s) : flash_h<false>(a, s);
}

// The reuse prefill keeps the tile's key list in dynamic LDS (k_max int32;
// over a paged cache also the k_max physical rows, so half as many keys).
size_t prefill_sparse_max_list() { return 24576; }
size_t prefill_sparse_paged_max_list() { return prefill_sparse_max_list() / 2; }

hipError_t prefill_set_max_lds() {
  const int bytes = (int)(prefill_sparse_max_list() * sizeof(int32_t));
  hipError_t e = set_lds_h<false, false>(bytes);
  if (e == hipSuccess) e = set_lds_h<true, false>(bytes);
  if (e == hipSuccess) e = set_lds_h<false, true>(bytes);
  if (e == hipSuccess) e = set_lds_h<true, true>(bytes);
  if (e == hipSuccess) e = set_pool_lds_h<false>();
  if (e == hipSuccess) e = set_pool_lds_h<true>();
  return e;
}

hipError_t launch_prefill_sparse(const PrefillArgs& a, hipStream_t s) {
  if (a.table) return a.half ? sparse_h<true, true>(a, s) : sparse_h<false, true>(a, s);
  return a.half ? sparse_h<true, false>(a, s) : sparse_h<false, false>(a, s);
}

hipError_t launch_prefill_pool(const PrefillArgs& a, hipStream_t s) {
  return a.half ? pool_h<true>(a, s) : pool_h<false>(a, s);
}

}  // namespace kc
