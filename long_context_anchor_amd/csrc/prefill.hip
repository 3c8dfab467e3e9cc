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

// One block of 64 keys held in registers between its global loads and its
// LDS store, so the loads of block i+1 are in flight while block i is used.
// K units: 64 rows x 16 chunks of 16 bytes, (kKB*16)/NT per thread.  V^T
// units: (16-key chunk, half, 4 d columns): 8 keys x 4 d, 256/NT per thread.
template <int NT, bool WITH_V>
struct KvRegs {
  static constexpr int KU = kKB * 16 / NT;
  static constexpr int VU = WITH_V ? 256 / NT : 0;
  uint4 k[KU];
  uint2 v[VU > 0 ? VU : 1][8];

  // pos(kr) gives the cache row of block row kr, or -1 for none.
  template <typename PosF>
  KC_INLINE void load(PosF pos, const char* kbase, const char* vbase, int64_t row_bytes) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + i * NT;
      const int p = pos(u >> 4);
      // always load (row 0 stands in for a missing row), then zero: no branch
      const uint4 x = ld16(kbase + (int64_t)(p < 0 ? 0 : p) * row_bytes + (u & 15) * 16);
      k[i] = p < 0 ? make_uint4(0, 0, 0, 0) : x;
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + i * NT;
      const int c4 = u >> 6, hp = (u >> 5) & 1, dg = u & 31;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int p = pos(c4 * 16 + 4 * hp + (s & 3) + 8 * (s >> 2));
        const uint2 x =
            *reinterpret_cast<const uint2*>(vbase + (int64_t)(p < 0 ? 0 : p) * row_bytes + dg * 8);
        v[i][s] = p < 0 ? make_uint2(0, 0) : x;
      }
    }
  }

  // K rows as [key][d] (padded); V^T as [d][key] with the keys of each
  // 16-key chunk in MFMA B-operand order (see the file comment).
  KC_INLINE void store(uint16_t* sk, uint16_t* svt) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + i * NT;
      sts16(sk + (u >> 4) * kKStride + (u & 15) * 8, k[i]);
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + i * NT;
      const int c4 = u >> 6, hp = (u >> 5) & 1, dg = u & 31;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t a[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) a[s] = (e < 2) ? v[i][s].x : v[i][s].y;
        uint4 o;
        o.x = __builtin_amdgcn_perm(a[1], a[0], sel);
        o.y = __builtin_amdgcn_perm(a[3], a[2], sel);
        o.z = __builtin_amdgcn_perm(a[5], a[4], sel);
        o.w = __builtin_amdgcn_perm(a[7], a[6], sel);
        sts16(svt + (dg * 4 + e) * kVStride + c4 * 16 + 8 * hp, o);
      }
    }
  }
};

struct __align__(16) AttnSmem {
  uint16_t k[kKB * kKStride];
  uint16_t vt[kD * kVStride];
};

// One workgroup = one (query tile, query head, batch); 4 waves x 32 rows.
// GATHER: the keys are the tile's list for KV head head_map[g] (ascending,
// staged in LDS once), masked per row by position <= row.
template <bool GATHER>
__global__ __launch_bounds__(256, 2) void k_prefill_attn(const PrefillArgs a) {
  __shared__ AttnSmem sm;
  extern __shared__ int32_t slist[];
  const int t = a.T - 1 - (int)blockIdx.x;   // longest causal tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
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
  if (GATHER) {
    nkeys = tile_k_for_len(P, a.pct, a.round_to, a.k_min);
    const int32_t* list = a.idx + ((int64_t)(b * a.T + t) * a.Hkv + a.hm.m[g]) * a.k_max;
    for (int i = tid; i < nkeys; i += 256) {
      const int p = list[i];
      slist[i] = (p >= 0 && p < N) ? p : -1;
    }
    __syncthreads();
  }
  const int64_t row_bytes = a.kv_sn * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh) * 2;
  auto pos_of = [&](int kb, int kr) -> int {
    const int i = kb + kr;
    if (i >= nkeys) return -1;
    return GATHER ? slist[i] : i;
  };

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m = kNegInf, l = 0.f;

  KvRegs<256, true> regs;
  regs.load([&](int kr) { return pos_of(0, kr); }, kbase, vbase, row_bytes);
  for (int kb = 0; kb < nkeys; kb += kKB) {
    __syncthreads();   // the previous block's LDS reads are done
    regs.store(sm.k, sm.vt);
    __syncthreads();
    if (kb + kKB < nkeys) regs.load([&](int kr) { return pos_of(kb + kKB, kr); }, kbase, vbase, row_bytes);

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
          s[kt][ri] = (p < 0 || p > r) ? kNegInf : s[kt][ri];
        }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) mx = fmaxf(mx, s[kt][ri]);
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
    const float mn = m;
    const bool live = mn != kNegInf;
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
  __shared__ float red[NW][kKB];

  const int t = a.T - 1 - (int)blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
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
    KvRegs<NT, false> regs;
    regs.load([&](int kr) { return kr < P ? kr : -1; }, kbase, nullptr, row_bytes);
    for (int kb = 0; kb < P; kb += kKB) {
      __syncthreads();
      regs.store(sk, nullptr);
      __syncthreads();
      if (kb + kKB < P)
        regs.load([&](int kr) { return kb + kKB + kr < P ? kb + kKB + kr : -1; }, kbase, nullptr,
                  row_bytes);
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
        if (need_mask) {
#pragma unroll
          for (int ri = 0; ri < 16; ++ri) {
            const int rr = row0 + 8 * (ri >> 2) + 4 * hf + (ri & 3);
            const float p = exp2f_fast(fmaf(acc[ri], c, -lse[ri]));
            cs += (j <= rr && rr < N && j < P) ? p : 0.f;
          }
        } else {
#pragma unroll
          for (int ri = 0; ri < 16; ++ri) cs += exp2f_fast(fmaf(acc[ri], c, -lse[ri]));
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

// The reuse prefill keeps the tile's key list in dynamic LDS (k_max int32).
size_t prefill_sparse_max_list() { return 24576; }

hipError_t prefill_set_max_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prefill_attn<true>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(prefill_sparse_max_list() * sizeof(int32_t)));
}

hipError_t launch_prefill_sparse(const PrefillArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.k_max * sizeof(int32_t);
  hipLaunchKernelGGL(k_prefill_attn<true>, dim3(a.T, a.Hq, a.B), dim3(256), lds, s, a);
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
