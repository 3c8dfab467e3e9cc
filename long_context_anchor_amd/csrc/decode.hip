// Decode kernels: split-K attention over a KV cache (dense anchor pass or
// gathered reuse pass), the split combine, and the head-aware pooling of the
// anchor's post-softmax probabilities.
//
// Method: the anchor layer computes full attention and keeps, per KV head,
// the post-softmax probabilities pooled over the head's query group; a reuse
// layer attends only to the keys of the anchor's list for KV head
// head_map[g] (page "論文解説: Kascade …", sections "アンカーレイヤーと再利用
// レイヤー" and "ヘッドリマッピング").
//
// Layout on gfx950.  One K/V row is 256 bytes (bf16 or fp16 x 128, fp32 x 64).  A
// 16-lane DPP row of a wave64 covers one K/V row with 16-byte loads, so one
// load instruction of a wave reads 4 consecutive rows (1 KiB contiguous).
// Each lane keeps its 16-byte slice of the group's G query heads in
// registers; a score is the 16-lane DPP sum of the lanes' partial dots, so K
// is read once for all G heads of the group.  Softmax runs in the log2
// domain (scale folded with log2(e), v_exp_f32).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "paged.h"
#include "radix.h"

namespace kc {

namespace {

constexpr int kThreads = 256;      // 4 waves
constexpr int kListPad = 64;       // LDS list entries past the split that a step may read
constexpr float kLazyLog2 = 8.f;   // slack of the lazily moved softmax reference (log2 units)
constexpr int kSpillPad = 16;      // per-head slack of the LDS score buffer

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int EPL = 4;    // fp32 per 16 bytes
  static constexpr int D = 64;
};
template <>
struct Elem<uint16_t> {
  static constexpr int D = 128;
};
template <>
struct Elem<_Float16> {
  static constexpr int D = 128;
};

// Partial dot of a 16-byte fp32 slice with a query slice (the fp32 kernel;
// 16-bit caches run the head-slot kernel below).
KC_INLINE float slice_dot(const uint4& kk, const uint4& qq, float acc, float) {
  acc = fmaf(__uint_as_float(kk.x), __uint_as_float(qq.x), acc);
  acc = fmaf(__uint_as_float(kk.y), __uint_as_float(qq.y), acc);
  acc = fmaf(__uint_as_float(kk.z), __uint_as_float(qq.z), acc);
  acc = fmaf(__uint_as_float(kk.w), __uint_as_float(qq.w), acc);
  return acc;
}
// Unpack a 16-byte fp32 slice.
KC_INLINE void slice_unpack(const uint4& w, float* f, float) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

// One workgroup = one (key split, KV head, batch).  It produces, for each of
// the G query heads of the group, the split's running max m (log2 domain),
// sum l = sum 2^(s-m) and o = sum 2^(s-m) v.
template <typename T, int G, bool GATHER, bool SPILL>
__global__ __launch_bounds__(kThreads) void k_decode_splitk(const DecodeArgs a) {
  constexpr int EPL = Elem<T>::EPL;
  constexpr int D = Elem<T>::D;
  // rows per lane-group per iteration: fewer for large groups to keep the
  // register footprint at two waves per SIMD
  constexpr int kRows = G >= 4 ? 8 : 16;
  constexpr int kWaveRows = 4 * kRows;
  __shared__ float s_m[4][G];
  __shared__ float s_l[4][G];
  __shared__ float s_o[4][G][D];
  extern __shared__ int32_t s_list[];   // GATHER: this split's key list

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gi = lane >> 4, li = lane & 15;
  const int k0 = split * a.keys_per_split;
  const int k1 = min(a.n_keys, k0 + a.keys_per_split);

  if (a.hist0 && split == 0) {
    const int64_t row = (int64_t)b * a.Hkv + g;
    uint32_t* h0 = a.hist0 + row * 2048;
    for (int i = tid; i < 2048; i += kThreads) h0[i] = 0u;
    if (a.hist1) {
      uint32_t* h1 = a.hist1 + row * 2048;
      for (int i = tid; i < 2048; i += kThreads) h1[i] = 0u;
    }
  }
  if (GATHER) {
    const int32_t* list = a.idx + (int64_t)b * a.idx_sb + (int64_t)a.hm.m[g] * a.idx_sg;
    for (int i = tid; i < k1 - k0; i += kThreads) s_list[i] = list[k0 + i];
    __syncthreads();
  }

  // query slices of the G heads of this group
  uint4 qs[G];
  for (int hh = 0; hh < G; ++hh) {
    const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.q_sb +
                  (int64_t)(g * G + hh) * a.q_sh;
    qs[hh] = ld16(reinterpret_cast<const char*>(qp) + li * 16);
  }
  const int64_t row_bytes = a.kv_sn * (int64_t)sizeof(T);
  const char* kb = reinterpret_cast<const char*>(a.k) +
                   ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * (int64_t)sizeof(T) + li * 16;
  const char* vb = reinterpret_cast<const char*>(a.v) +
                   ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * (int64_t)sizeof(T) + li * 16;

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNegInf;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  }

  // each wave takes a contiguous quarter of the split (a multiple of the 4
  // rows one load instruction covers), so the waves finish together
  const int per_wave = ((k1 - k0 + 15) >> 4) << 2;
  const int w0 = k0 + wave * per_wave;
  const int w1 = min(k1, w0 + per_wave);
  for (int c = w0; c < w1; c += kWaveRows) {
    uint4 kr[kRows], vr[kRows];
    bool ok[kRows];
#pragma unroll
    for (int t = 0; t < kRows; ++t) {
      const int r = c + 4 * t + gi;
      ok[t] = r < w1;
      // gathered positions are clamped into the cache so a bad list cannot fault
      int64_t j = GATHER ? (ok[t] ? min(max(s_list[r - k0], 0), a.n_ctx - 1) : 0) : r;
      kr[t] = ok[t] ? ld16(kb + j * row_bytes) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kRows; ++t) {
      const int r = c + 4 * t + gi;
      int64_t j = GATHER ? (ok[t] ? min(max(s_list[r - k0], 0), a.n_ctx - 1) : 0) : r;
      vr[t] = ok[t] ? ld16(vb + j * row_bytes) : make_uint4(0, 0, 0, 0);
    }
    float sc[G][kRows];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int t = 0; t < kRows; ++t) {
        float d = row16_sum(slice_dot(kr[t], qs[hh], 0.f, T()));
        sc[hh][t] = ok[t] ? d * a.scale_log2 : kNegInf;
      }
    }
    if (SPILL) {
      // lane li writes the score of row t = li: consecutive floats per wave
      const int r = c + 4 * li + gi;
      if (li < kRows && r < w1) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float mine = sc[hh][0];
#pragma unroll
          for (int t = 1; t < kRows; ++t) mine = (li == t) ? sc[hh][t] : mine;
          a.scores[((int64_t)b * a.Hq + g * G + hh) * a.n_keys + r] = mine;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float cm = sc[hh][0];
#pragma unroll
      for (int t = 1; t < kRows; ++t) cm = fmaxf(cm, sc[hh][t]);
      const float mn = fmaxf(m[hh], cm);
      const float alpha = (mn == kNegInf) ? 0.f : exp2f_fast(m[hh] - mn);
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] *= alpha;
      m[hh] = mn;
    }
#pragma unroll
    for (int t = 0; t < kRows; ++t) {
      float vf[EPL];
      slice_unpack(vr[t], vf, T());
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = ok[t] ? exp2f_fast(sc[hh][t] - m[hh]) : 0.f;
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(p, vf[e], o[hh][e]);
      }
    }
  }

  // merge the 4 lane-groups of each wave (lanes li, li+16, li+32, li+48 hold
  // the same output slice), then the 4 waves through LDS
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float M = fmaxf(m[hh], __shfl_xor(m[hh], 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    const float w = (M == kNegInf) ? 0.f : exp2f_fast(m[hh] - M);
    float L = l[hh] * w;
    L += __shfl_xor(L, 16, 64);
    L += __shfl_xor(L, 32, 64);
    m[hh] = M;
    l[hh] = L;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = o[hh][e] * w;
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      o[hh][e] = x;
    }
  }
  if (gi == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (li == 0) {
        s_m[wave][hh] = m[hh];
        s_l[wave][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][hh][li * EPL + e] = o[hh][e];
    }
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int hh = x / D, dd = x % D;
    float M = kNegInf;
    for (int q = 0; q < 4; ++q) M = fmaxf(M, s_m[q][hh]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
      for (int q = 0; q < 4; ++q) {
        const float w = exp2f_fast(s_m[q][hh] - M);
        L = fmaf(s_l[q][hh], w, L);
        O = fmaf(s_o[q][hh][dd], w, O);
      }
    }
    float* pp = a.part + (((int64_t)b * a.Hq + g * G + hh) * a.n_splits + split) * (D + 2);
    pp[2 + dd] = O;
    if (dd == 0) {
      pp[0] = M;
      pp[1] = L;
    }
  }
}

// ---- 16-bit (bf16 / fp16) split-K kernel with head slots -------------------------
//
// The same work as k_decode_splitk for 16-bit caches, laid out so that the
// per-row softmax runs once per head instead of once per head per lane.
// Lane li of a 16-lane row "owns" head own = li / (16/G) of the group and
// keeps its partial dots in slot order: slot k holds head k ^ own.  A
// reduce-scatter over the row (mirror, half mirror, xor 2, xor 1) then
// leaves every lane with the full score of its own head for the row.  The
// probabilities of the other heads come back through the same lane
// exchanges, and P.V runs on pairs of rows with v_dot2c_f32_bf16 / _f16 (P
// rounded to the cache's type, fp32 accumulation), so a row costs 16 dot2 for the scores, 5 DPP
// adds, one exp and 16 dot2 for the output per lane.

// Lane moves within 16-lane rows; every control used here reads a lane of
// the same row, so bound_ctrl never applies and no old value is needed.
template <int CTRL>
KC_INLINE uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_XOR3 = 0x1B;    // quad_perm [3,2,1,0]
constexpr int DPP_ROR8 = 0x128;   // row_ror:8, lane i <- i ^ 8 within 16 lanes

// Value of a lane of the same 16-lane row whose own head is ours ^ K
// (LG = log2 G).  Own heads are li >> (4 - LG), so any lane li ^ X with
// X >> (4 - LG) == K will do; each case picks one or two DPP moves.
template <int K, int LG>
KC_INLINE uint32_t slot_xchg(uint32_t v) {
  static_assert(K >= 1 && K < (1 << LG), "slot exchange");
  if constexpr (LG == 1) {
    return dpp_u<DPP_MIRROR>(v);                            // X = 15
  } else if constexpr (LG == 2) {
    if constexpr (K == 1) return dpp_u<DPP_HALF_MIRROR>(v);  // X = 7
    else if constexpr (K == 2) return dpp_u<DPP_ROR8>(v);    // X = 8
    else return dpp_u<DPP_MIRROR>(v);                        // X = 15
  } else {
    if constexpr (K == 1) return dpp_u<DPP_XOR2>(v);                              // X = 2
    else if constexpr (K == 2) return dpp_u<DPP_XOR3>(dpp_u<DPP_HALF_MIRROR>(v));  // X = 4
    else if constexpr (K == 3) return dpp_u<DPP_HALF_MIRROR>(v);                  // X = 7
    else if constexpr (K == 4) return dpp_u<DPP_ROR8>(v);                         // X = 8
    else if constexpr (K == 5) return dpp_u<DPP_XOR2>(dpp_u<DPP_ROR8>(v));         // X = 10
    else if constexpr (K == 6) return dpp_u<DPP_XOR3>(dpp_u<DPP_MIRROR>(v));       // X = 12
    else return dpp_u<DPP_MIRROR>(v);                                              // X = 15
  }
}
// Reduce-scatter of G slot partials over a 16-lane row: returns, in every
// lane, the row sum of the lane's own head (slot 0).
template <int G>
KC_INLINE float reduce_scatter(float (&s)[G]) {
  constexpr int F0 = G - 1, F1 = (G - 1) >> 1, F2 = (G - 1) >> 2;
  if constexpr (F0 > 0) {
#pragma unroll
    for (int k = 0; k < G / 2; ++k) s[k] += dpp_f<DPP_MIRROR>(s[k ^ F0]);
  } else {
    s[0] += dpp_f<DPP_MIRROR>(s[0]);
  }
  if constexpr (F1 > 0) {
#pragma unroll
    for (int k = 0; k < G / 4; ++k) s[k] += dpp_f<DPP_HALF_MIRROR>(s[k ^ F1]);
  } else {
    s[0] += dpp_f<DPP_HALF_MIRROR>(s[0]);
  }
  if constexpr (F2 > 0) {
    s[0] += dpp_f<DPP_XOR2>(s[1]);
  } else {
    s[0] += dpp_f<DPP_XOR2>(s[0]);
  }
  s[0] += dpp_f<DPP_XOR1>(s[0]);
  return s[0];
}

template <int G, int LG, int K = 1>
KC_INLINE void slots_from_own(uint32_t own_v, uint32_t (&out)[G]) {
  if constexpr (K == 1) out[0] = own_v;
  if constexpr (K < G) {
    out[K] = slot_xchg<K, LG>(own_v);
    slots_from_own<G, LG, K + 1>(own_v, out);
  }
}

// The split-K pass of one workgroup up to its four waves' partial states in
// LDS (s_m, s_l, s_o per wave and head).  KEEP: the split's scores stay in
// LDS (s_list, after the row list when paged) instead of being written out.
template <int G, bool GATHER, bool SPILL, bool PAGED, bool HALF, int kRows, bool KEEP>
KC_INLINE void splitk_slots_core(const DecodeArgs& a, int32_t* s_list, float (&s_m)[4][G],
                                 float (&s_l)[4][G], float (&s_o)[4][G][128]) {
  typedef Fmt16<HALF> F;   // bf16 or fp16 elements
  constexpr int LG = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  static_assert(kRows % 4 == 0, "list entries are read four at a time");
  constexpr int kWaveRows = 4 * kRows;  // rows per wave per step
  // the split's rows go through an LDS list when they are gathered or paged
  constexpr bool LIST = GATHER || PAGED;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gi = lane >> 4, li = lane & 15;
  const int own = li >> (4 - LG);
  const int k0 = split * a.keys_per_split;
  const int k1 = min(a.n_keys, k0 + a.keys_per_split);

  if (a.hist0 && split == 0) {
    const int64_t row = (int64_t)b * a.Hkv + g;
    uint32_t* h0 = a.hist0 + row * 2048;
    for (int i = tid; i < 2048; i += kThreads) h0[i] = 0u;
    if (a.hist1) {
      uint32_t* h1 = a.hist1 + row * 2048;
      for (int i = tid; i < 2048; i += kThreads) h1[i] = 0u;
    }
  }
  if (LIST) {
    const int32_t* list = a.idx + (int64_t)b * a.idx_sb + (int64_t)a.hm.m[g] * a.idx_sg;
    for (int i = tid; i < k1 - k0; i += kThreads) {
      int j = GATHER ? list[k0 + i] : k0 + i;
      // logical position -> physical row (positions and blocks clamped so a
      // bad list or table cannot fault)
      if (PAGED)
        j = (int)paged_row(a.table, a.table_stride, b, j, a.n_ctx, a.blk_shift, a.num_blocks,
                           (uint32_t)a.blk_rows);
      s_list[i] = j;
    }
    // a step may read up to 15 entries past the split's rows: make them row 0
    for (int i = (k1 - k0) + tid; i < (k1 - k0) + kListPad; i += kThreads) s_list[i] = 0;
    __syncthreads();
  }

  // query slices in slot order: slot k = head k ^ own of the group
  uint4 qs[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_sb +
                         (int64_t)(g * G + (k ^ own)) * a.q_sh;
    qs[k] = ld16(reinterpret_cast<const char*>(qp) + li * 16);
  }
  // 32-bit byte offsets from the head's base (the host keeps a head under
  // 4 GiB); paged caches use 64-bit offsets of physical rows
  const uint32_t row_bytes = (uint32_t)a.kv_sn * (uint32_t)sizeof(uint16_t);
  const int64_t head_off =
      ((PAGED ? 0 : (int64_t)b * a.kv_sb) + (int64_t)g * a.kv_sh) * (int64_t)sizeof(uint16_t);
  // last valid row: head g's rows of the last block end at row bs-1 (the
  // head offset is added to every row address)
  const uint32_t max_row = PAGED ? paged_max_row(a.num_blocks, (uint32_t)a.blk_rows, a.blk_shift)
                                 : (uint32_t)(a.n_ctx - 1);
  const char* kbase = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.v) + head_off;
  const uint32_t lane_off = (uint32_t)li * 16u;

  float m = kNegInf, l = 0.f;   // own head
  float o[G][8];                // slot k: head k ^ own, elements 8 li .. 8 li + 7
#pragma unroll
  for (int k = 0; k < G; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[k][e] = 0.f;

  // Score spill (anchor pass): one lane per (head, lane group) keeps the
  // group's scores in LDS ([G][kps + kSpillPad]); the split's scores leave in
  // one coalesced burst after the loop.  Stores issued inside the loop would
  // share vmcnt with the K/V loads and hold up every following wait.
  float* const s_sc = reinterpret_cast<float*>(s_list) + (PAGED ? a.keys_per_split + kListPad : 0);

  // each wave takes a contiguous quarter of the split; in a step, lane group
  // gi takes kRows consecutive rows
  const int per_wave = ((k1 - k0 + 15) >> 4) << 2;
  const int w0 = k0 + wave * per_wave;
  const int w1 = min(k1, w0 + per_wave);
  for (int c = w0; c < w1; c += kWaveRows) {
    const bool full = c + kWaveRows <= w1;   // uniform over the wave
    const int r0 = c + kRows * gi;
    typedef typename std::conditional<PAGED, uint64_t, uint32_t>::type off_t;
    off_t off[kRows];
    if (LIST) {
      // entries past w1 are read (the LDS list is padded) and replaced below
#pragma unroll
      for (int t4 = 0; t4 < kRows; t4 += 4) {
        const int4 j4 = *reinterpret_cast<const int4*>(s_list + (r0 + t4 - k0));
        const int jj[4] = {j4.x, j4.y, j4.z, j4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // rows are clamped into the cache so a bad list cannot fault
          const uint32_t j = PAGED ? min((uint32_t)jj[u], max_row) : (uint32_t)min(max(jj[u], 0), (int)max_row);
          off[t4 + u] = (off_t)j * row_bytes + lane_off;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kRows; ++t) off[t] = (uint32_t)min(r0 + t, w1 - 1) * row_bytes + lane_off;
    }
    // K/V rows are read once per call: nontemporal loads keep them from
    // displacing reusable lines in the caches (measured 7-10% faster at 128K)
    uint4 kr[kRows], vr[kRows];
#pragma unroll
    for (int t = 0; t < kRows; ++t) kr[t] = ld16_nt(kbase + off[t]);
#pragma unroll
    for (int t = 0; t < kRows; ++t) vr[t] = ld16_nt(vbase + off[t]);
    if (!full) {
      // rows past the end: their V must not meet p = 0 as inf/nan
#pragma unroll
      for (int t = 0; t < kRows; ++t)
        if (r0 + t >= w1) vr[t] = make_uint4(0, 0, 0, 0);
    }

    float sc[kRows];
#pragma unroll
    for (int t = 0; t < kRows; ++t) {
      float part[G];
#pragma unroll
      for (int k = 0; k < G; ++k)
        part[k] = F::dot2(kr[t].w, qs[k].w, F::dot2(kr[t].z, qs[k].z,
                  F::dot2(kr[t].y, qs[k].y, F::dot2(kr[t].x, qs[k].x, 0.f))));
      sc[t] = reduce_scatter<G>(part) * a.scale_log2;
    }
    if (!full) {
#pragma unroll
      for (int t = 0; t < kRows; ++t) sc[t] = (r0 + t < w1) ? sc[t] : kNegInf;
    }
    if (SPILL && (li & ((16 >> LG) - 1)) == 0) {
      // rows past w1 belong to the next wave's range and are not written
      float* dst = s_sc + own * (a.keys_per_split + kSpillPad) + (r0 - k0);
      if (full) {
#pragma unroll
        for (int t4 = 0; t4 < kRows; t4 += 4)
          *reinterpret_cast<float4*>(dst + t4) = make_float4(sc[t4], sc[t4 + 1], sc[t4 + 2], sc[t4 + 3]);
      } else {
#pragma unroll
        for (int t = 0; t < kRows; ++t)
          if (r0 + t < w1) dst[t] = sc[t];
      }
    }
    // Lazy rescaling: the reference max m only moves when a score exceeds it
    // by more than kLazyLog2 (so p <= 2^kLazyLog2), and the rescale of the
    // accumulators runs only in steps where some lane of the wave moves.
    float cm = sc[0];
#pragma unroll
    for (int t = 1; t < kRows; ++t) cm = fmaxf(cm, sc[t]);
    const bool move = cm > m + kLazyLog2;   // false while both are -inf
    if (__any(move)) {
      const float mn = move ? cm : m;
      const float alpha = (mn == kNegInf) ? 1.f : exp2f_fast(m - mn);
      m = mn;
      l *= alpha;
      uint32_t al[G];
      slots_from_own<G, LG>(__float_as_uint(alpha), al);
#pragma unroll
      for (int k = 0; k < G; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[k][e] *= __uint_as_float(al[k]);
    }
    float p[kRows];
    if (full && m != kNegInf) {
#pragma unroll
      for (int t = 0; t < kRows; ++t) p[t] = exp2f_fast(sc[t] - m);
    } else {
#pragma unroll
      for (int t = 0; t < kRows; ++t) p[t] = (sc[t] == kNegInf) ? 0.f : exp2f_fast(sc[t] - m);
    }
#pragma unroll
    for (int t = 0; t < kRows; ++t) l += p[t];
#pragma unroll
    for (int t = 0; t < kRows; t += 2) {
      uint32_t pk[G];
      slots_from_own<G, LG>(F::pack(p[t], p[t + 1]), pk);
      const uint32_t w0v[4] = {vr[t].x, vr[t].y, vr[t].z, vr[t].w};
      const uint32_t w1v[4] = {vr[t + 1].x, vr[t + 1].y, vr[t + 1].z, vr[t + 1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // (row t, row t+1) pairs of elements 2j and 2j+1
        const uint32_t ev = __builtin_amdgcn_perm(w1v[j], w0v[j], 0x05040100u);
        const uint32_t od = __builtin_amdgcn_perm(w1v[j], w0v[j], 0x07060302u);
#pragma unroll
        for (int k = 0; k < G; ++k) {
          o[k][2 * j] = F::dot2(ev, pk[k], o[k][2 * j]);
          o[k][2 * j + 1] = F::dot2(od, pk[k], o[k][2 * j + 1]);
        }
      }
    }
  }

  if (SPILL && !KEEP) {
    __syncthreads();
    const int n = k1 - k0;
    for (int hh = 0; hh < G; ++hh) {
      const float* src = s_sc + hh * (a.keys_per_split + kSpillPad);
      float* dst = a.scores + ((int64_t)b * a.Hq + g * G + hh) * a.n_keys + k0;
      const int nv = (a.n_keys & 3) == 0 ? (n & ~3) : 0;   // 16-byte rows only
      for (int i = tid * 4; i < nv; i += kThreads * 4)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(src + i),
                                    reinterpret_cast<f32x4_t*>(dst + i));
      for (int i = nv + tid; i < n; i += kThreads) __builtin_nontemporal_store(src[i], dst + i);
    }
  }

  // Merge the 4 lane groups of each wave (rows gi of the wave; lanes li,
  // li+16, li+32, li+48 own the same head and output slice) with
  // v_permlane32_swap / v_permlane16_swap: for swap(a, b) the two results
  // add up to a[l] + a[l^32] in lanes 0..31 and b[l^32] + b[l] in lanes
  // 32..63 (rows of 16 lanes for the 16-lane swap).  Max and sums are
  // exchanged in full; the G*8 output values are reduce-scattered in two
  // halvings, after which lane (gi, li) holds values gi*2G .. gi*2G+2G-1 of
  // its slot-major list (slot k, element e at k*8+e).
  {
    auto swap32 = [](float x, float y) {
      return __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    };
    auto swap16 = [](float x, float y) {
      return __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    };
    auto r0 = [](auto r) { return __uint_as_float(r[0]); };
    auto r1 = [](auto r) { return __uint_as_float(r[1]); };
    auto s32 = swap32(m, m);
    float M = fmaxf(r0(s32), r1(s32));
    auto s16 = swap16(M, M);
    M = fmaxf(r0(s16), r1(s16));
    const float w = (M == kNegInf) ? 0.f : exp2f_fast(m - M);
    float L = l * w;
    s32 = swap32(L, L);
    L = r0(s32) + r1(s32);
    s16 = swap16(L, L);
    L = r0(s16) + r1(s16);
    uint32_t ws[G];
    slots_from_own<G, LG>(__float_as_uint(w), ws);
    constexpr int N = 8 * G;
    float v[N];
#pragma unroll
    for (int k = 0; k < G; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k * 8 + e] = o[k][e] * __uint_as_float(ws[k]);
#pragma unroll
    for (int n = 0; n < N / 2; ++n) {
      const auto r = swap32(v[n], v[n + N / 2]);
      v[n] = r0(r) + r1(r);
    }
#pragma unroll
    for (int n = 0; n < N / 4; ++n) {
      const auto r = swap16(v[n], v[n + N / 4]);
      v[n] = r0(r) + r1(r);
    }
    // value n is list entry n + gi * N/4: slot (n + gi*N/4) / 8, element % 8
    if (li % (16 >> LG) == 0 && gi == 0) {
      s_m[wave][own] = M;
      s_l[wave][own] = L;
    }
#pragma unroll
    for (int n = 0; n < N / 4; n += 2) {
      const int idx = n + gi * (N / 4);
      const int k = idx >> 3, e = idx & 7;
      *reinterpret_cast<float2*>(&s_o[wave][k ^ own][li * 8 + e]) = make_float2(v[n], v[n + 1]);
    }
  }
}

template <int G, bool GATHER, bool SPILL, bool PAGED = false, bool HALF = false, int kRows = 4>
__global__ __launch_bounds__(kThreads) void k_decode_splitk_slots(const DecodeArgs a) {
  constexpr int D = 128;
  __shared__ float s_m[4][G];
  __shared__ float s_l[4][G];
  __shared__ float s_o[4][G][D];
  // dynamic LDS: the row list (kps + kListPad entries: cache positions, or
  // physical row numbers when paged), then the spilled scores
  extern __shared__ __align__(16) int32_t s_list[];
  splitk_slots_core<G, GATHER, SPILL, PAGED, HALF, kRows, false>(a, s_list, s_m, s_l, s_o);
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int hh = x / D, dd = x % D;
    float M = kNegInf;
    for (int q = 0; q < 4; ++q) M = fmaxf(M, s_m[q][hh]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
      for (int q = 0; q < 4; ++q) {
        const float w = exp2f_fast(s_m[q][hh] - M);
        L = fmaf(s_l[q][hh], w, L);
        O = fmaf(s_o[q][hh][dd], w, O);
      }
    }
    float* pp = a.part + (((int64_t)b * a.Hq + g * G + hh) * a.n_splits + split) * (D + 2);
    pp[2 + dd] = O;
    if (dd == 0) {
      pp[0] = M;
      pp[1] = L;
    }
  }
}

// Merge the splits of query head bh with NT threads: thread (part, dd) folds
// splits part, part + PARTS, ... into a running (max, sum, output column dd)
// with kBatch splits' loads issued up front, then the PARTS partial states of
// each column meet once in LDS (sm, sl, so hold NT floats each) and threads
// < D write the normalised column; thread 0 writes the lse.
// Words exchanged between the workgroups of one launch (the fused anchor
// decode): relaxed atomics at agent scope, which the compiler issues for
// gfx950 as global stores and loads with the sc1 (device scope) bit and no
// cache writeback or invalidate instructions; the hardware keeps such
// accesses coherent across the device.
KC_INLINE void st_coh(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
KC_INLINE void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
KC_INLINE float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
KC_INLINE uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COH>
KC_INLINE float ld_part(const float* p) {
  if constexpr (COH) return ld_coh(p);
  else return *p;
}

template <typename T, int NT, int kBatch, bool COH = false>
KC_INLINE void merge_splits(const float* part, int S, int64_t bh, void* out, float* lse2,
                            float* lse_out, float* sm, float* sl, float* so) {
  constexpr int D = Elem<T>::D;
  constexpr int PARTS = NT / D;
  const int tid = threadIdx.x;
  const int dd = tid % D, prt = tid / D;
  const float* p = part + bh * S * (D + 2);

  float M = kNegInf, L = 0.f, O = 0.f;
  for (int s0 = prt; s0 < S; s0 += PARTS * kBatch) {
    float mv[kBatch], lv[kBatch], ov[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + u * PARTS;
      const float* ps = p + (int64_t)min(s, S - 1) * (D + 2);
      mv[u] = s < S ? ld_part<COH>(ps) : kNegInf;
      lv[u] = ld_part<COH>(ps + 1);
      ov[u] = ld_part<COH>(ps + 2 + dd);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float mn = fmaxf(M, mv[u]);
      if (mn == kNegInf) continue;   // nothing seen yet (empty splits)
      const float sc = exp2f_fast(M - mn), w = exp2f_fast(mv[u] - mn);
      L = fmaf(L, sc, lv[u] * w);
      O = fmaf(O, sc, ov[u] * w);
      M = mn;
    }
  }
  sm[prt * D + dd] = M;
  sl[prt * D + dd] = L;
  so[prt * D + dd] = O;
  __syncthreads();
  if (tid < D) {
    float Mt = kNegInf;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) Mt = fmaxf(Mt, sm[q * D + tid]);
    float Lt = 0.f, Ot = 0.f;
    if (Mt != kNegInf) {
#pragma unroll
      for (int q = 0; q < PARTS; ++q) {
        const float w = exp2f_fast(sm[q * D + tid] - Mt);
        Lt = fmaf(sl[q * D + tid], w, Lt);
        Ot = fmaf(so[q * D + tid], w, Ot);
      }
    }
    const float r = Lt > 0.f ? Ot / Lt : 0.f;
    if constexpr (std::is_same<T, _Float16>::value) {
      reinterpret_cast<_Float16*>(out)[bh * D + tid] = (_Float16)r;
    } else if constexpr (sizeof(T) == 2) {
      reinterpret_cast<uint16_t*>(out)[bh * D + tid] = (uint16_t)f32_to_bf16_bits(r);
    } else {
      reinterpret_cast<float*>(out)[bh * D + tid] = r;
    }
    if (tid == 0) {
      const float l2 = Mt + log2f_fast(Lt);
      if (lse2) lse2[bh] = l2;
      if (lse_out) lse_out[bh] = l2 * kLn2;
    }
  }
}

// One workgroup per (batch, query head): merge the splits (reuse and dense
// passes).
constexpr int kCombineThreads = 1024;
constexpr int kMaxSplits = 2048;

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void k_decode_combine(const CombineArgs a) {
  __shared__ float sm[kCombineThreads], sl[kCombineThreads], so[kCombineThreads];
  merge_splits<T, kCombineThreads, 8>(a.part, a.n_splits, blockIdx.x, a.out, a.lse2, a.lse_out, sm,
                                      sl, so);
}

// (M, L) += (Mo, Lo) in the log2 domain: the larger maximum, the sums
// rescaled to it.
KC_INLINE void lse_merge(float& M, float& L, float Mo, float Lo) {
  const float mn = fmaxf(M, Mo);
  L = mn == kNegInf ? 0.f : fmaf(L, exp2f_fast(M - mn), Lo * exp2f_fast(Mo - mn));
  M = mn;
}

// The (M, L) pairs of a wave's 64 lanes merged into lane 0 (the other lanes
// end with partial merges): across the halves and the 16-lane rows with the
// lane-swap instructions (both lanes of a pair see the lower lane's value
// first), then inside each row with DPP mirrors and quad permutes.  No LDS.
KC_INLINE void wave_lse_reduce(float& M, float& L) {
  const auto m32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(M), __float_as_uint(M), false, false);
  const auto l32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(L), __float_as_uint(L), false, false);
  M = __uint_as_float(m32[0]);
  L = __uint_as_float(l32[0]);
  lse_merge(M, L, __uint_as_float(m32[1]), __uint_as_float(l32[1]));
  const auto m16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(M), __float_as_uint(M), false, false);
  const auto l16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(L), __float_as_uint(L), false, false);
  M = __uint_as_float(m16[0]);
  L = __uint_as_float(l16[0]);
  lse_merge(M, L, __uint_as_float(m16[1]), __uint_as_float(l16[1]));
  lse_merge(M, L, dpp_f<DPP_MIRROR>(M), dpp_f<DPP_MIRROR>(L));
  lse_merge(M, L, dpp_f<DPP_HALF_MIRROR>(M), dpp_f<DPP_HALF_MIRROR>(L));
  lse_merge(M, L, dpp_f<DPP_XOR2>(M), dpp_f<DPP_XOR2>(L));
  lse_merge(M, L, dpp_f<DPP_XOR1>(M), dpp_f<DPP_XOR1>(L));
}

// Anchor pooling fused with the anchor pass's split merge (see
// PoolDecodeArgs).  A pooling workgroup issues its 1024 keys' score loads for
// the G heads of KV head g, merges the heads' lse from the splits' (m, l)
// (wave w takes heads w, w + 4) while those loads are in flight, then writes
// pooled[j] = sum_h 2^(s_hj - lse_h) and the digit-0 histogram of the row.
template <typename T, int G>
__global__ __launch_bounds__(256) void k_decode_pool(const PoolDecodeArgs a) {
  constexpr int D = Elem<T>::D;
  __shared__ uint32_t sh[2048];
  __shared__ float s_lse[G];
  __shared__ float sm[256], sl[256], so[256];
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int chunks = (a.N + 1023) / 1024;
  if ((int)blockIdx.x >= chunks) {   // merge workgroup of query head g*G + (x - chunks)
    const int64_t bh = (int64_t)b * a.Hq + g * G + ((int)blockIdx.x - chunks);
    merge_splits<T, 256, 16>(a.part, a.n_splits, bh, a.out, nullptr, a.lse_out, sm, sl, so);
    return;
  }
  for (int i = tid; i < 2048; i += 256) sh[i] = 0u;
  const int j = (blockIdx.x * 256 + tid) * 4;
  const float* sp[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) sp[hh] = a.scores + ((int64_t)b * a.Hq + g * G + hh) * a.N;
  const bool vec = j + 4 <= a.N && (a.N & 3) == 0;
  float4 s4[G];
  if (vec) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s4[hh] = *reinterpret_cast<const float4*>(sp[hh] + j);
  }
  {
    const int wave = tid >> 6, lane = tid & 63;
    for (int hh = wave; hh < G; hh += 4) {
      const float* p = a.part + ((int64_t)b * a.Hq + g * G + hh) * a.n_splits * (D + 2);
      float M = kNegInf, L = 0.f;
      for (int s = lane; s < a.n_splits; s += 64) {
        const float m = p[(int64_t)s * (D + 2)], l = p[(int64_t)s * (D + 2) + 1];
        const float mn = fmaxf(M, m);
        if (mn != kNegInf) {
          L = fmaf(L, exp2f_fast(M - mn), l * exp2f_fast(m - mn));
          M = mn;
        }
      }
      wave_lse_reduce(M, L);
      if (lane == 0) s_lse[hh] = M + log2f_fast(L);
    }
  }
  __syncthreads();
  float lse[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) lse[hh] = s_lse[hh];
  float* out = a.pooled + ((int64_t)b * a.Hkv + g) * a.N;
  if (j < a.N) {
    if (vec) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        acc.x += exp2f_fast(s4[hh].x - lse[hh]);
        acc.y += exp2f_fast(s4[hh].y - lse[hh]);
        acc.z += exp2f_fast(s4[hh].z - lse[hh]);
        acc.w += exp2f_fast(s4[hh].w - lse[hh]);
      }
      *reinterpret_cast<float4*>(out + j) = acc;
      atomicAdd(&sh[f32_order_key(acc.x) >> 21], 1u);
      atomicAdd(&sh[f32_order_key(acc.y) >> 21], 1u);
      atomicAdd(&sh[f32_order_key(acc.z) >> 21], 1u);
      atomicAdd(&sh[f32_order_key(acc.w) >> 21], 1u);
    } else {
      for (int jj = j; jj < min(a.N, j + 4); ++jj) {
        float acc = 0.f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) acc += exp2f_fast(sp[hh][jj] - lse[hh]);
        out[jj] = acc;
        atomicAdd(&sh[f32_order_key(acc) >> 21], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* h0 = a.hist0 + ((int64_t)b * a.Hkv + g) * 2048;
  for (int i = tid; i < 2048; i += 256) {
    const uint32_t c = sh[i];
    if (c) atomicAdd(&h0[i], c);
  }
}

// ---- fused anchor decode --------------------------------------------------
//
// One launch per anchor layer: grid (splits, Hkv, B) of workgroups that are
// all resident at once (the host checks the grid against the GPU's resident
// slots).  A row = the splits of one (batch, KV head).
//   phase 1  the split-K pass of the split (scores kept in LDS); its
//            partial (m, l, o) per head is published; split 0 clears the
//            row's two histograms;                          -> row barrier 1
//   phase 2  every workgroup merges the row's (m, l) into each head's lse,
//            pools its keys' probabilities over the G heads into order keys
//            (LDS) and adds its digit-0 histogram to the row's; arrives;
//            split s then merges the splits of query heads s, s + S, ... of
//            the group into out / lse_out;                  -> row barrier 2
//   phase 3  digit 0's bin b0 from the row histogram; the split's keys above
//            b0 are counted and its keys in b0 (the candidates) stored at its
//            own offset, with their digit-1 histogram added to the row's;
//                                                           -> row barrier 3
//   phase 4  digits 1 and 2 fix the k-th largest key T and how many keys
//            equal to T are taken; the counts of the earlier splits give the
//            split's output offset; its indices are written in index order.
// A barrier is a per-row counter: each workgroup adds one after its
// exchanged stores are complete (vmcnt 0) and thread 0 polls the counter a
// bounded number of times; a workgroup that gives up sets status bit 0 and
// skips its remaining phases (it still arrives, so the others are not held
// longer).  The last workgroup of the row to leave clears the row's counters.

// Thread 0 adds the workgroup to the row's barrier once every thread's
// exchanged stores have completed.
KC_INLINE void row_arrive(uint32_t* ctr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the row's counter reaches target; false (uniform over the
// workgroup) if thread 0 gave up after `limit` polls.
KC_INLINE bool row_wait(const uint32_t* ctr, uint32_t target, uint32_t limit, uint32_t* status,
                        uint32_t* s_ok) {
  if (threadIdx.x == 0) {
    uint32_t ok = 1u, n = 0;
    while (ld_coh(ctr) < target) {
      if (++n > limit) {
        ok = 0u;
        atomicOr(status, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0u;
}

// Candidate f of the row in split order: its split by binary search over the
// exclusive prefix of the splits' candidate counts, then its key.
KC_INLINE uint32_t fused_cand(const uint32_t* cand_row, const uint32_t* cpre, int S, int kps, uint32_t f) {
  int lo = 0, hi = S - 1;   // last split whose prefix is <= f
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cpre[mid] <= f) lo = mid;
    else hi = mid - 1;
  }
  return ld_coh(cand_row + (int64_t)lo * kps + (f - cpre[lo]));
}

template <int G, bool HALF>
__global__ __launch_bounds__(kThreads) void k_anchor_fused(const FusedDecodeArgs f) {
  typedef typename std::conditional<HALF, _Float16, uint16_t>::type T;
  constexpr int D = 128;
  constexpr int NB = 2048;
  __shared__ float s_m[4][G];
  __shared__ float s_l[4][G];
  __shared__ float s_o[4][G][D];
  __shared__ uint32_t s_hist[NB];          // histograms; merge scratch in phase 2
  __shared__ uint32_t s_cpre[kThreads];    // exclusive prefix of the splits' candidate counts
  __shared__ uint32_t sh[8], s_sel[2], s_ok;
  __shared__ float s_lse[G];
  extern __shared__ __align__(16) int32_t s_list[];   // scores [G][kps + kSpillPad]
  const DecodeArgs& a = f.d;

  splitk_slots_core<G, false, true, false, HALF, 4, true>(a, s_list, s_m, s_l, s_o);

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int S = a.n_splits, kps = a.keys_per_split, N = a.n_keys;
  const int k0 = split * kps;
  const int n = min(N, k0 + kps) - k0;
  const int64_t row = (int64_t)b * a.Hkv + g;
  uint32_t* ctr = f.sync + row * kFusedSyncWords;
  uint32_t* h0 = f.hist0 + row * NB;
  uint32_t* h1 = f.hist1 + row * NB;
  uint32_t* cand_row = f.cand + row * N;
  uint32_t* cnt_row = f.cnt + row * S * 2;
  float* sc = reinterpret_cast<float*>(s_list);
  uint32_t* keys = reinterpret_cast<uint32_t*>(s_list);   // order keys over head 0's scores
  const int sstride = kps + kSpillPad;
  __syncthreads();

  // phase 1: the split's partial state per head (as the split-K epilogue)
  for (int x = tid; x < G * D; x += kThreads) {
    const int hh = x / D, dd = x % D;
    float M = kNegInf;
    for (int q = 0; q < 4; ++q) M = fmaxf(M, s_m[q][hh]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
      for (int q = 0; q < 4; ++q) {
        const float w = exp2f_fast(s_m[q][hh] - M);
        L = fmaf(s_l[q][hh], w, L);
        O = fmaf(s_o[q][hh][dd], w, O);
      }
    }
    float* pp = a.part + (((int64_t)b * a.Hq + g * G + hh) * S + split) * (D + 2);
    st_coh(pp + 2 + dd, O);
    if (dd == 0) {
      st_coh(pp, M);
      st_coh(pp + 1, L);
    }
  }
  if (split == 0) {
    for (int i = tid; i < NB; i += kThreads) {
      st_coh(h0 + i, 0u);
      st_coh(h1 + i, 0u);
    }
  }
  row_arrive(ctr);
  bool ok = row_wait(ctr, (uint32_t)S, f.spin_limit, f.status, &s_ok);

  // phase 2: lse of the group's heads (wave w: heads w, w + 4), pooled keys
  // and the digit-0 histogram (the same arithmetic as the pooling kernel)
  if (ok) {
    const int wave = tid >> 6, lane = tid & 63;
    for (int hh = wave; hh < G; hh += 4) {
      const float* p = a.part + ((int64_t)b * a.Hq + g * G + hh) * S * (D + 2);
      float M = kNegInf, L = 0.f;
      for (int s2 = lane; s2 < S; s2 += 64) {
        const float m = ld_coh(p + (int64_t)s2 * (D + 2)), l = ld_coh(p + (int64_t)s2 * (D + 2) + 1);
        const float mn = fmaxf(M, m);
        if (mn != kNegInf) {
          L = fmaf(L, exp2f_fast(M - mn), l * exp2f_fast(m - mn));
          M = mn;
        }
      }
      wave_lse_reduce(M, L);
      if (lane == 0) s_lse[hh] = M + log2f_fast(L);
    }
    for (int i = tid; i < NB; i += kThreads) s_hist[i] = 0u;
    __syncthreads();
    float lse[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) lse[hh] = s_lse[hh];
    float* pooled = f.pooled ? f.pooled + row * N + k0 : nullptr;
    for (int i = tid; i < n; i += kThreads) {
      float acc = 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) acc += exp2f_fast(sc[hh * sstride + i] - lse[hh]);
      const uint32_t key = f32_order_key(acc);
      keys[i] = key;   // head 0's score i was read by this thread only
      if (pooled) pooled[i] = acc;
      atomicAdd(&s_hist[key >> 21], 1u);
    }
    __syncthreads();
    for (int i = tid; i < NB; i += kThreads) {
      const uint32_t c = s_hist[i];
      if (c) atomicAdd(&h0[i], c);
    }
  }
  row_arrive(ctr);
  if (ok) {
    // split s merges heads s, s + S, ... of the group (a row may have fewer
    // splits than heads)
    float* scratch = reinterpret_cast<float*>(s_hist);
    for (int hh = split; hh < G; hh += S) {
      merge_splits<T, kThreads, 16, true>(a.part, S, (int64_t)b * a.Hq + g * G + hh, f.out, nullptr,
                                          f.lse_out, scratch, scratch + kThreads, scratch + 2 * kThreads);
      __syncthreads();   // the scratch is rewritten by the next head
    }
  }
  ok = ok && row_wait(ctr, 2u * S, f.spin_limit, f.status, &s_ok);

  // phase 3: digit 0's bin; the split's keys above it and its candidates
  uint32_t b0 = 0, above0 = 0;
  const int R = (n + kThreads - 1) / kThreads;   // consecutive keys per thread
  const int i0 = tid * R;
  if (ok) {
    for (int i = tid; i < NB; i += kThreads) s_hist[i] = ld_coh(h0 + i);
    __syncthreads();
    b0 = find_bin256<NB>(s_hist, (uint32_t)f.k, sh, s_sel, above0);
    for (int i = tid; i < NB; i += kThreads) s_hist[i] = 0u;
    __syncthreads();
    uint32_t cn = 0, hi = 0;
    for (int q = 0; q < R; ++q) {
      const int i = i0 + q;
      if (i < n) {
        const uint32_t key = keys[i], d0 = key >> 21;
        if (d0 == b0) {
          atomicAdd(&s_hist[(key >> 10) & 2047u], 1u);
          ++cn;
        }
        hi += d0 > b0 ? 1u : 0u;
      }
    }
    uint32_t tot;
    const uint32_t off = scan256((cn << 16) | hi, sh, tot);
    uint32_t* cp = cand_row + k0 + (off >> 16);
    for (int q = 0; q < R; ++q) {
      const int i = i0 + q;
      if (i < n && (keys[i] >> 21) == b0) st_coh(cp++, keys[i]);
    }
    if (tid == 0) {
      st_coh(cnt_row + 2 * split, tot & 0xFFFFu);
      st_coh(cnt_row + 2 * split + 1, tot >> 16);
    }
    __syncthreads();
    for (int i = tid; i < NB; i += kThreads) {
      const uint32_t c = s_hist[i];
      if (c) atomicAdd(&h1[i], c);
    }
  }
  row_arrive(ctr);
  ok = ok && row_wait(ctr, 3u * S, f.spin_limit, f.status, &s_ok);

  // phase 4: the threshold key T and the split's indices
  if (ok) {
    uint32_t need = (uint32_t)f.k - above0, above;
    // the splits' counts (one split per thread; counts clamped to the split),
    // loaded together with the row's digit-1 histogram
    uint32_t nc = 0, ab = 0;
    if (tid < S) {
      const uint32_t len = (uint32_t)min(kps, N - tid * kps);
      nc = min(ld_coh(cnt_row + 2 * tid + 1), len);
      ab = tid < split ? min(ld_coh(cnt_row + 2 * tid), len) : 0u;
    }
    for (int i = tid; i < NB; i += kThreads) s_hist[i] = ld_coh(h1 + i);
    __syncthreads();
    const uint32_t b1 = find_bin256<NB>(s_hist, need, sh, s_sel, above);
    need -= above;
    const uint32_t p01 = (b0 << 11) | b1;
    uint32_t ncand, above_before, nc_ex, ab_ex;
    scan256x2(nc, ab, sh, nc_ex, ab_ex, ncand, above_before);
    s_cpre[tid] = nc_ex;
    for (int i = tid; i < 1024; i += kThreads) s_hist[i] = 0u;
    __syncthreads();   // s_cpre is read by every thread below
    // The row's candidates, copied into the free part of the LDS score buffer
    // when they fit (the two passes below then read LDS): thread t copies the
    // flat range [t*RC, t*RC + RC), eight coherent loads in flight at a time.
    uint32_t* s_cand = keys + kps;
    const bool staged = ncand <= f.cand_cap;
    if (staged) {
      const uint32_t RC = (ncand + kThreads - 1) / kThreads;
      const uint32_t c0 = tid * RC, c1 = min(ncand, c0 + RC);
      if (c0 < c1) {
        int sp = 0, hi = S - 1;   // last split whose prefix is <= c0
        while (sp < hi) {
          const int mid = (sp + hi + 1) >> 1;
          if (s_cpre[mid] <= c0) sp = mid;
          else hi = mid - 1;
        }
        uint32_t off = c0 - s_cpre[sp];
        for (uint32_t c = c0; c < c1; c += 8) {
          uint32_t v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            v[u] = 0u;
            if (c + u < c1) {
              // skip splits whose candidates are used up (or that have none)
              while (sp + 1 < S && s_cpre[sp] + off >= s_cpre[sp + 1]) {
                ++sp;
                off = 0;
              }
              v[u] = ld_coh(cand_row + (int64_t)sp * kps + off);
              ++off;
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (c + u < c1) s_cand[c + u] = v[u];
        }
      }
    }
    __syncthreads();
    auto cand_at = [&](uint32_t c) {
      return staged ? s_cand[c] : fused_cand(cand_row, s_cpre, S, kps, c);
    };
    for (uint32_t c = tid; c < ncand; c += kThreads) {
      const uint32_t key = cand_at(c);
      if ((key >> 10) == p01) atomicAdd(&s_hist[key & 1023u], 1u);
    }
    __syncthreads();
    const uint32_t b2 = find_bin256<1024>(s_hist, need, sh, s_sel, above);
    need -= above;
    const uint32_t Tk = (p01 << 10) | b2;   // the k-th largest key; `need` keys == Tk are taken
    const uint32_t cend = s_cpre[split];
    uint32_t gtc = 0, eqc = 0;
    for (uint32_t c = tid; c < cend; c += kThreads) {
      const uint32_t key = cand_at(c);
      gtc += key > Tk ? 1u : 0u;
      eqc += key == Tk ? 1u : 0u;
    }
    uint32_t gtc_ex, eqc_ex, gt_before, eq_before;
    scan256x2(gtc, eqc, sh, gtc_ex, eqc_ex, gt_before, eq_before);   // block totals
    gt_before += above_before;
    uint32_t gt = 0, eq = 0;
    for (int q = 0; q < R; ++q) {
      const int i = i0 + q;
      if (i < n) {
        gt += keys[i] > Tk ? 1u : 0u;
        eq += keys[i] == Tk ? 1u : 0u;
      }
    }
    uint32_t tot;
    const uint32_t ex = scan256((gt << 16) | eq, sh, tot);
    uint32_t g2 = gt_before + (ex >> 16), e2 = eq_before + (ex & 0xFFFFu);
    int32_t* out = f.idx + row * f.k;
    const uint32_t kk = (uint32_t)f.k;
    for (int q = 0; q < R; ++q) {
      const int i = i0 + q;
      if (i < n) {
        const uint32_t key = keys[i];
        if (key > Tk) {
          const uint32_t pos = g2 + min(e2, need);
          if (pos < kk) out[pos] = k0 + i;
          ++g2;
        } else if (key == Tk) {
          if (e2 < need && g2 + e2 < kk) out[g2 + e2] = k0 + i;
          ++e2;
        }
      }
    }
  }

  // leave: the row's last workgroup clears its counters for the next call
  __syncthreads();
  if (tid == 0) {
    const uint32_t t = __hip_atomic_fetch_add(ctr + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t + 1 == (uint32_t)S) {
      st_coh(ctr, 0u);
      st_coh(ctr + 32, 0u);
    }
  }
}

// 16-bit caches run the head-slot kernel, fp32 caches the plain one (which
// has no paged variant: the host rejects paged fp32).
template <typename T, int G, bool GATHER, bool SPILL, bool PAGED = false>
constexpr void (*splitk_kernel())(const DecodeArgs) {
  if constexpr (sizeof(T) == 2)
    return k_decode_splitk_slots<G, GATHER, SPILL, PAGED, std::is_same<T, _Float16>::value>;
  else return k_decode_splitk<T, G, GATHER, SPILL>;
}

template <typename T, int G, bool PAGED>
void (*splitk_pick(bool gather, bool spill))(const DecodeArgs) {
  return gather ? splitk_kernel<T, G, true, false, PAGED>()
         : spill ? splitk_kernel<T, G, false, true, PAGED>()
                 : splitk_kernel<T, G, false, false, PAGED>();
}

template <typename T, int G>
hipError_t splitk_attrs_t(bool gather, bool spill, bool paged, int* blocks, size_t* static_lds) {
  void (*k)(const DecodeArgs) = paged ? splitk_pick<T, G, true>(gather, spill)
                                      : splitk_pick<T, G, false>(gather, spill);
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, (const void*)k);
  if (e != hipSuccess) return e;
  *static_lds = fa.sharedSizeBytes;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, kThreads, 0);
}

template <typename T>
hipError_t splitk_attrs_g(int G, bool gather, bool spill, bool paged, int* blocks,
                          size_t* static_lds) {
  switch (G) {
    case 1: return splitk_attrs_t<T, 1>(gather, spill, paged, blocks, static_lds);
    case 2: return splitk_attrs_t<T, 2>(gather, spill, paged, blocks, static_lds);
    case 4: return splitk_attrs_t<T, 4>(gather, spill, paged, blocks, static_lds);
    case 8: return splitk_attrs_t<T, 8>(gather, spill, paged, blocks, static_lds);
  }
  return hipErrorInvalidValue;
}

// Largest dynamic LDS of a 16-bit spilling launch: the score buffer of the
// longest split (or the one-workgroup-per-CU floor), plus the row list when
// the cache is paged.
inline size_t spill_dyn_lds_cap(bool paged) {
  const size_t most = paged ? kSpillMaxLds : kSpillMaxLdsOne;
  const size_t scores = most > kSpillMinLds ? most : kSpillMinLds;
  return scores + (paged ? (kPlanMaxKeys + kListPad) * sizeof(int32_t) : 0);
}

template <int G, bool HALF>
hipError_t spill_set_lds_gh() {
  hipError_t e = hipFuncSetAttribute((const void*)k_decode_splitk_slots<G, false, true, false, HALF>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)spill_dyn_lds_cap(false));
  if (e != hipSuccess) return e;
  // the dense pass with long splits asks for the one-workgroup-per-CU floor
  e = hipFuncSetAttribute((const void*)k_decode_splitk_slots<G, false, false, false, HALF>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSpillMinLds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)k_decode_splitk_slots<G, false, true, true, HALF>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)spill_dyn_lds_cap(true));
}
template <int G>
hipError_t spill_set_lds_g() {
  hipError_t e = spill_set_lds_gh<G, false>();
  return e != hipSuccess ? e : spill_set_lds_gh<G, true>();
}

template <typename T, int G>
hipError_t launch_splitk_t(const DecodeArgs& a, bool gather, hipStream_t s) {
  if (a.n_splits > kMaxSplits || a.n_splits < 1) return hipErrorInvalidValue;
  const bool paged = a.table != nullptr;
  if (paged && sizeof(T) != 2) return hipErrorInvalidValue;
  if ((gather || paged) && a.keys_per_split > kMaxGatherKeys) return hipErrorInvalidValue;
  const bool spill = !gather && a.scores;
  const size_t lds = decode_splitk_dyn_lds(sizeof(T) == 2 ? 1 : 0, G, gather, spill, paged,
                                           a.keys_per_split);
  if (spill && lds > spill_dyn_lds_cap(paged))
    return hipErrorInvalidValue;
  dim3 grid(a.n_splits, a.Hkv, a.B);
  void (*k)(const DecodeArgs) = paged ? splitk_pick<T, G, true>(gather, spill)
                                      : splitk_pick<T, G, false>(gather, spill);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_splitk_g(const DecodeArgs& a, bool gather, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_splitk_t<T, 1>(a, gather, s);
    case 2: return launch_splitk_t<T, 2>(a, gather, s);
    case 4: return launch_splitk_t<T, 4>(a, gather, s);
    case 8: return launch_splitk_t<T, 8>(a, gather, s);
  }
  return hipErrorInvalidValue;
}

template <int G, bool HALF>
hipError_t fused_launch_gh(const FusedDecodeArgs& f, hipStream_t s) {
  const size_t lds = anchor_fused_dyn_lds(G, f.d.keys_per_split);
  hipLaunchKernelGGL((k_anchor_fused<G, HALF>), dim3(f.d.n_splits, f.d.Hkv, f.d.B), dim3(kThreads), lds, s, f);
  return hipGetLastError();
}

template <bool HALF>
hipError_t fused_launch_h(const FusedDecodeArgs& f, hipStream_t s) {
  switch (f.d.Hq / f.d.Hkv) {
    case 1: return fused_launch_gh<1, HALF>(f, s);
    case 2: return fused_launch_gh<2, HALF>(f, s);
    case 4: return fused_launch_gh<4, HALF>(f, s);
    case 8: return fused_launch_gh<8, HALF>(f, s);
  }
  return hipErrorInvalidValue;
}

template <int G, bool HALF>
hipError_t fused_attrs_gh(int kps, int* blocks, size_t* static_lds) {
  const void* k = reinterpret_cast<const void*>(&k_anchor_fused<G, HALF>);
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, k);
  if (e != hipSuccess) return e;
  *static_lds = fa.sharedSizeBytes;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, kThreads, anchor_fused_dyn_lds(G, kps));
}

template <bool HALF>
hipError_t fused_attrs_h(int G, int kps, int* blocks, size_t* static_lds) {
  switch (G) {
    case 1: return fused_attrs_gh<1, HALF>(kps, blocks, static_lds);
    case 2: return fused_attrs_gh<2, HALF>(kps, blocks, static_lds);
    case 4: return fused_attrs_gh<4, HALF>(kps, blocks, static_lds);
    case 8: return fused_attrs_gh<8, HALF>(kps, blocks, static_lds);
  }
  return hipErrorInvalidValue;
}

// The fused kernel's dynamic LDS may grow to the spill cap or to what its
// static LDS leaves of the CU's 160 KiB, whichever is smaller.
template <int G, bool HALF>
hipError_t fused_set_lds_gh() {
  const void* k = reinterpret_cast<const void*>(&k_anchor_fused<G, HALF>);
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, k);
  if (e != hipSuccess) return e;
  const size_t room = fa.sharedSizeBytes < kLdsPerCu ? kLdsPerCu - fa.sharedSizeBytes : 0;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(room < kSpillMaxLdsOne ? room : kSpillMaxLdsOne));
}
template <int G>
hipError_t fused_set_lds_g() {
  hipError_t e = fused_set_lds_gh<G, false>();
  return e != hipSuccess ? e : fused_set_lds_gh<G, true>();
}

}  // namespace

size_t spill_lds_bytes(int G, int keys_per_split) {
  return (size_t)G * (size_t)(keys_per_split + kSpillPad) * sizeof(float);
}

int spill_max_keys(int G, bool paged) {
  const size_t lds = paged ? kSpillMaxLds : kSpillMaxLdsOne;
  const int cap = paged ? kPlanMaxKeys : kSpillMaxKeysOne;
  const int k = (int)(lds / ((size_t)G * sizeof(float))) - kSpillPad;
  return (k < cap ? k : cap) & ~15;
}

hipError_t decode_set_max_lds() {
  hipError_t e;
  if ((e = spill_set_lds_g<1>()) != hipSuccess) return e;
  if ((e = spill_set_lds_g<2>()) != hipSuccess) return e;
  if ((e = spill_set_lds_g<4>()) != hipSuccess) return e;
  if ((e = spill_set_lds_g<8>()) != hipSuccess) return e;
  if ((e = fused_set_lds_g<1>()) != hipSuccess) return e;
  if ((e = fused_set_lds_g<2>()) != hipSuccess) return e;
  if ((e = fused_set_lds_g<4>()) != hipSuccess) return e;
  return fused_set_lds_g<8>();
}

// Dynamic LDS of the fused anchor decode: the split's scores, with the same
// one-workgroup-per-CU floor as the spilling pass.
size_t anchor_fused_dyn_lds(int G, int kps) {
  const size_t b = spill_lds_bytes(G, kps);
  return b < kSpillMinLds ? kSpillMinLds : b;
}

hipError_t anchor_fused_attrs(int dtype, int G, int kps, int* blocks, size_t* static_lds) {
  return dtype == 2 ? fused_attrs_h<true>(G, kps, blocks, static_lds)
                    : fused_attrs_h<false>(G, kps, blocks, static_lds);
}

hipError_t launch_anchor_fused(const FusedDecodeArgs& f, int dtype, hipStream_t s) {
  if (f.d.n_splits < 1 || f.d.n_splits > kThreads || f.d.keys_per_split > kSpillMaxKeysOne)
    return hipErrorInvalidValue;
  return dtype == 2 ? fused_launch_h<true>(f, s) : fused_launch_h<false>(f, s);
}

hipError_t decode_splitk_attrs(int dtype, int G, bool gather, bool spill, bool paged, int* blocks,
                               size_t* static_lds) {
  if (dtype == 2) return splitk_attrs_g<_Float16>(G, gather, spill, paged, blocks, static_lds);
  return dtype == 1 ? splitk_attrs_g<uint16_t>(G, gather, spill, paged, blocks, static_lds)
                    : splitk_attrs_g<float>(G, gather, spill, paged, blocks, static_lds);
}

size_t decode_splitk_dyn_lds(int dtype, int G, bool gather, bool spill, bool paged, int kps) {
  size_t bytes = (gather || paged) ? (size_t)(kps + kListPad) * sizeof(int32_t) : 0;
  if (spill && dtype != 0) {
    bytes += spill_lds_bytes(G, kps);
    if (bytes < kSpillMinLds) bytes = kSpillMinLds;   // one spilling workgroup per CU
  }
  if (!spill && !gather && !paged && dtype != 0 && kps >= kDenseOneWgKeys && bytes < kSpillMinLds)
    bytes = kSpillMinLds;   // long dense splits: one workgroup per CU too
  return bytes;
}

hipError_t launch_decode_splitk(const DecodeArgs& a, int dtype, bool gather, hipStream_t s) {
  if (dtype == 2) return launch_splitk_g<_Float16>(a, gather, s);
  return dtype == 1 ? launch_splitk_g<uint16_t>(a, gather, s) : launch_splitk_g<float>(a, gather, s);
}

hipError_t launch_decode_combine(const CombineArgs& a, int dtype, hipStream_t s) {
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  if (dtype == 2)
    hipLaunchKernelGGL(k_decode_combine<_Float16>, dim3(a.BH), dim3(kCombineThreads), 0, s, a);
  else if (dtype == 1)
    hipLaunchKernelGGL(k_decode_combine<uint16_t>, dim3(a.BH), dim3(kCombineThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_decode_combine<float>, dim3(a.BH), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pool_t(const PoolDecodeArgs& a, hipStream_t s) {
  dim3 grid((a.N + 1023) / 1024 + a.Hq / a.Hkv, a.Hkv, a.B);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((k_decode_pool<T, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_decode_pool<T, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_decode_pool<T, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_decode_pool<T, 8>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_pool(const PoolDecodeArgs& a, int dtype, hipStream_t s) {
  if (a.n_splits > kMaxSplits || a.n_splits < 1) return hipErrorInvalidValue;
  if (dtype == 2) return launch_pool_t<_Float16>(a, s);
  return dtype == 1 ? launch_pool_t<uint16_t>(a, s) : launch_pool_t<float>(a, s);
}

}  // namespace kc
