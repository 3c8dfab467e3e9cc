// Prefill kernels (bf16, head_dim 128, 128-query tiles) on gfx950 MFMA.
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
//                          2^(S*c - lse2) over the G heads x 128 rows
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, wave64).  Operand A is 32x16 with
// lane l holding row l%32, k = 8*(l/32)..+7; operand B is 16x32 with lane l
// holding column l%32, the same k; the 32x32 fp32 result gives lane l column
// l%32 and rows 8i + 4*(l/32) + j in register 4i+j.
//   attention: S^T = K Q^T (A = K rows from LDS, B = Q rows in registers),
//     so each lane owns one query and its softmax row statistics stay in
//     the lane (plus its partner lane l^32).  P^T in that C layout is
//     already the B operand of O^T = V^T P^T once the key order of a
//     16-key chunk is permuted; V is written to LDS transposed in that
//     permuted order so the A operand is one 16-byte LDS read.
//   pooling: S = Q K^T (A = Q registers, B = K from LDS), so each lane owns
//     one key column and the pooled column sum is an in-lane sum.
#include "common.h"
#include "kernels.h"

namespace kc {

namespace {

constexpr int kD = 128;
constexpr int kTileQ = 128;            // query rows per tile (4 waves x 32)
constexpr int kKB = 64;                // keys per block
constexpr int kKStride = kD + 8;       // bf16 per K row in LDS (272 B: conflict-free reads)
constexpr int kVStride = kKB + 8;      // bf16 per V^T row in LDS (144 B)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

KC_INLINE bf16x8_t as_bf16x8(const uint4& u) {
  u32x4 v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8_t, v);
}
KC_INLINE uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
KC_INLINE void sts16(uint16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

KC_INLINE f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Stage one block of 64 K rows ([key][d], padded) and V^T ([d][key],
// permuted within 16-key chunks) into LDS.  pos[] holds the block's key
// positions (-1 = none).  NT threads.
template <int NT>
KC_INLINE void stage_kv(uint16_t* sk, uint16_t* svt, const int32_t* pos, const char* kbase,
                        const char* vbase, int64_t row_bytes, bool with_v) {
  const int tid = threadIdx.x;
  // K: 64 rows x 16 chunks of 16 bytes
#pragma unroll
  for (int u = tid; u < kKB * 16; u += NT) {
    const int kr = u >> 4, ch = u & 15;
    const int p = pos[kr];
    uint4 val = make_uint4(0, 0, 0, 0);
    if (p >= 0) val = ld16(kbase + (int64_t)p * row_bytes + ch * 16);
    sts16(sk + kr * kKStride + ch * 8, val);
  }
  if (!with_v) return;
  // V^T: unit = (16-key chunk c4, half hp, 4 d columns dg); 8 keys x 4 d each
#pragma unroll
  for (int u = tid; u < 256; u += NT) {
    const int c4 = u >> 6, hp = (u >> 5) & 1, dg = u & 31;
    uint2 w[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kr = c4 * 16 + 4 * hp + (s & 3) + 8 * (s >> 2);
      const int p = pos[kr];
      w[s] = make_uint2(0, 0);
      if (p >= 0) w[s] = *reinterpret_cast<const uint2*>(vbase + (int64_t)p * row_bytes + dg * 8);
    }
    // column e of the 4: element e of every key, packed two keys per word
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint4 o;
      const uint32_t a0 = (e < 2) ? w[0].x : w[0].y, a1 = (e < 2) ? w[1].x : w[1].y;
      const uint32_t a2 = (e < 2) ? w[2].x : w[2].y, a3 = (e < 2) ? w[3].x : w[3].y;
      const uint32_t a4 = (e < 2) ? w[4].x : w[4].y, a5 = (e < 2) ? w[5].x : w[5].y;
      const uint32_t a6 = (e < 2) ? w[6].x : w[6].y, a7 = (e < 2) ? w[7].x : w[7].y;
      o.x = __builtin_amdgcn_perm(a1, a0, sel);
      o.y = __builtin_amdgcn_perm(a3, a2, sel);
      o.z = __builtin_amdgcn_perm(a5, a4, sel);
      o.w = __builtin_amdgcn_perm(a7, a6, sel);
      sts16(svt + (dg * 4 + e) * kVStride + c4 * 16 + 8 * hp, o);
    }
  }
}

struct __align__(16) AttnSmem {
  uint16_t k[kKB * kKStride];
  uint16_t vt[kD * kVStride];
  int32_t pos[kKB];
};

// One workgroup = one (query tile, query head, batch); 4 waves x 32 rows.
template <bool GATHER>
__global__ __launch_bounds__(256) void k_prefill_attn(const PrefillArgs a) {
  __shared__ AttnSmem sm;
  const int t = a.T - 1 - (int)blockIdx.x;   // longest causal tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int N = a.N;
  const int row0 = t * kTileQ + wave * 32;
  const int r = row0 + l32;
  const float c = a.scale_log2;

  // queries as the B operand: lane holds row r, d = 16*ds + 8*hf + 0..7
  bf16x8_t qf[8];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)min(r, N - 1) * a.q_sn) * 2;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (r < N) u = ld16(qp + (ds * 16 + hf * 8) * 2);
      qf[ds] = as_bf16x8(u);
    }
  }
  const int P = min(N, kTileQ * (t + 1));
  int nkeys = P;
  const int32_t* list = nullptr;
  if (GATHER) {
    nkeys = tile_k_for_len(P, a.pct, a.round_to, a.k_min);
    list = a.idx + ((int64_t)(b * a.T + t) * a.Hkv + a.hm.m[g]) * a.k_max;
  }
  const int64_t row_bytes = a.kv_sn * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * 2;

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  for (int kb = 0; kb < nkeys; kb += kKB) {
    __syncthreads();   // the previous block's LDS reads are done
    if (tid < kKB) {
      int p = -1;
      if (kb + tid < nkeys) {
        p = GATHER ? list[kb + tid] : kb + tid;
        p = (p >= 0 && p < N) ? p : -1;
      }
      sm.pos[tid] = p;
    }
    __syncthreads();
    stage_kv<256>(sm.k, sm.vt, sm.pos, kbase, vbase, row_bytes, true);
    __syncthreads();

    f32x16_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16_t{};
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const bf16x8_t kf = as_bf16x8(lds16(sm.k + (kt * 32 + l32) * kKStride + ds * 16 + hf * 8));
        s[kt] = mfma32(kf, qf[ds], s[kt]);
      }
    }
    // causal mask inside the block (key position > query row) and empty slots
    bool need_mask;
    if (GATHER) {
      need_mask = (kb + kKB > nkeys) || (sm.pos[kKB - 1] > row0) || (sm.pos[kKB - 1] < 0);
    } else {
      need_mask = (kb + kKB - 1 > row0) || (kb + kKB > nkeys);
    }
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        if (need_mask) {
          const int kr = kt * 32 + 8 * (ri >> 2) + 4 * hf + (ri & 3);
          const int p = sm.pos[kr];
          if (p < 0 || p > r) s[kt][ri] = kNegInf;
        }
        mx = fmaxf(mx, s[kt][ri]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx * c);
    const bool live = mn != kNegInf;
    const float alpha = live ? exp2f_fast(m - mn) : 1.f;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= alpha;
    m = mn;
    // P^T (bf16) as the B operand of O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = live ? exp2f_fast(fmaf(s[kt][8 * c2 + e], c, -mn)) : 0.f;
          l += p[e];
        }
        uint4 pk;
        pk.x = pack_bf16x2(p[0], p[1]);
        pk.y = pack_bf16x2(p[2], p[3]);
        pk.z = pack_bf16x2(p[4], p[5]);
        pk.w = pack_bf16x2(p[6], p[7]);
        const bf16x8_t pb = as_bf16x8(pk);
        const int chunk = kt * 2 + c2;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8_t vf =
              as_bf16x8(lds16(sm.vt + (db * 32 + l32) * kVStride + chunk * 16 + hf * 8));
          o[db] = mfma32(vf, pb, o[db]);
        }
      }
    }
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
        w.x = pack_bf16x2(o[db][4 * i + 0] * inv, o[db][4 * i + 1] * inv);
        w.y = pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
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

// One workgroup = one (query tile, KV head, batch): 4*WH waves; wave w takes
// the 32-row slice w%4 of the tile for heads (w/4) + WH*i of the group, one
// head at a time (i outer), so a wave holds one head's queries.
template <int G>
__global__ __launch_bounds__(256 * (G < 4 ? G : 4)) void k_prefill_pool(const PrefillArgs a) {
  constexpr int WH = G < 4 ? G : 4;          // head lanes of waves
  constexpr int HPW = G / WH;                // heads per wave
  constexpr int NT = 256 * WH;
  constexpr int NW = NT / 64;
  __shared__ __align__(16) uint16_t sk[kKB * kKStride];
  __shared__ int32_t spos[kKB];
  __shared__ float red[NW][kKB];

  const int t = a.T - 1 - (int)blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int slice = wave & 3, hw = wave >> 2;
  const int N = a.N;
  const int row0 = t * kTileQ + slice * 32;
  const float c = a.scale_log2;
  const int P = min(N, kTileQ * (t + 1));
  const int64_t row_bytes = a.kv_sn * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * 2;
  float* prow = a.pooled + (int64_t)b * a.packed_per_batch + packed_row_offset(t, g, a.Hkv, kTileQ, N);

  for (int hi = 0; hi < HPW; ++hi) {
    bf16x8_t qf[8];
    float lse[16];
    {
      const int h = g * G + hw + WH * hi;
      const int r = row0 + l32;
      const char* qp = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)min(r, N - 1) * a.q_sn) * 2;
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (r < N) u = ld16(qp + (ds * 16 + hf * 8) * 2);
        qf[ds] = as_bf16x8(u);
      }
      const float* lp = a.lse2 + ((int64_t)b * a.Hq + h) * N;
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        const int rr = row0 + 8 * (ri >> 2) + 4 * hf + (ri & 3);
        lse[ri] = rr < N ? lp[rr] : 0.f;
      }
    }
    for (int kb = 0; kb < P; kb += kKB) {
      __syncthreads();
      if (tid < kKB) spos[tid] = (kb + tid < P) ? kb + tid : -1;
      __syncthreads();
      stage_kv<NT>(sk, nullptr, spos, kbase, nullptr, row_bytes, false);
      __syncthreads();
      const bool need_mask = (kb + kKB - 1 > row0) || (kb + kKB > P) || (row0 + 32 > N);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16_t acc = f32x16_t{};
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
          const bf16x8_t kf = as_bf16x8(lds16(sk + (kt * 32 + l32) * kKStride + ds * 16 + hf * 8));
          acc = mfma32(qf[ds], kf, acc);
        }
        const int j = kb + kt * 32 + l32;
        float cs = 0.f;
#pragma unroll
        for (int ri = 0; ri < 16; ++ri) {
          float p = exp2f_fast(fmaf(acc[ri], c, -lse[ri]));
          if (need_mask) {
            const int rr = row0 + 8 * (ri >> 2) + 4 * hf + (ri & 3);
            p = (j <= rr && rr < N && j < P) ? p : 0.f;
          }
          cs += p;
        }
        cs += __shfl_xor(cs, 32, 64);
        if (hf == 0) red[wave][kt * 32 + l32] = cs;
      }
      __syncthreads();
      if (tid < kKB && kb + tid < P) {
        float sum = hi == 0 ? 0.f : prow[kb + tid];
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w][tid];
        prow[kb + tid] = sum;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_flash(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_prefill_attn<false>, dim3(a.T, a.Hq, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_sparse(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_prefill_attn<true>, dim3(a.T, a.Hq, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_pool(const PrefillArgs& a, hipStream_t s) {
  dim3 grid(a.T, a.Hkv, a.B);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL(k_prefill_pool<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_prefill_pool<2>, grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_prefill_pool<4>, grid, dim3(1024), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_prefill_pool<8>, grid, dim3(1024), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kc
