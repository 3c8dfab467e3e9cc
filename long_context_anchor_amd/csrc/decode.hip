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
// Layout on gfx950.  One K/V row is 256 bytes (bf16 x 128 or fp32 x 64).  A
// 16-lane DPP row of a wave64 covers one K/V row with 16-byte loads, so one
// load instruction of a wave reads 4 consecutive rows (1 KiB contiguous).
// Each lane keeps its 16-byte slice of the group's G query heads in
// registers; a score is the 16-lane DPP sum of the lanes' partial dots, so K
// is read once for all G heads of the group.  Softmax runs in the log2
// domain (scale folded with log2(e), v_exp_f32).
#include "common.h"
#include "kernels.h"

namespace kc {

namespace {

constexpr int kThreads = 256;      // 4 waves

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int EPL = 4;    // fp32 per 16 bytes
  static constexpr int D = 64;
};
template <>
struct Elem<uint16_t> {
  static constexpr int EPL = 8;    // bf16 per 16 bytes
  static constexpr int D = 128;
};

// Partial dot of a 16-byte slice with a query slice.
KC_INLINE float slice_dot(const uint4& kk, const uint4& qq, float acc, uint16_t) {
  acc = dot2_bf16(kk.x, qq.x, acc);
  acc = dot2_bf16(kk.y, qq.y, acc);
  acc = dot2_bf16(kk.z, qq.z, acc);
  acc = dot2_bf16(kk.w, qq.w, acc);
  return acc;
}
KC_INLINE float slice_dot(const uint4& kk, const uint4& qq, float acc, float) {
  acc = fmaf(__uint_as_float(kk.x), __uint_as_float(qq.x), acc);
  acc = fmaf(__uint_as_float(kk.y), __uint_as_float(qq.y), acc);
  acc = fmaf(__uint_as_float(kk.z), __uint_as_float(qq.z), acc);
  acc = fmaf(__uint_as_float(kk.w), __uint_as_float(qq.w), acc);
  return acc;
}
// Unpack a 16-byte slice to fp32.
KC_INLINE void slice_unpack(const uint4& w, float* f, uint16_t) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
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
  constexpr int kBlockRows = 4 * kWaveRows;
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
    uint32_t* h0 = a.hist0 + ((int64_t)b * a.Hkv + g) * 2048;
    for (int i = tid; i < 2048; i += kThreads) h0[i] = 0u;
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

  for (int c = k0 + wave * kWaveRows; c < k1; c += kBlockRows) {
    uint4 kr[kRows], vr[kRows];
    bool ok[kRows];
#pragma unroll
    for (int t = 0; t < kRows; ++t) {
      const int r = c + 4 * t + gi;
      ok[t] = r < k1;
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
      if (li < kRows && r < k1) {
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

// One workgroup per (batch, query head): merge the splits.  The split
// weights 2^(m_s - M) are formed once in LDS; every thread then sums a
// strided share of the splits for one output column (independent loads).
constexpr int kCombineThreads = 256;
constexpr int kMaxSplits = 2048;

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void k_decode_combine(const CombineArgs a) {
  constexpr int D = Elem<T>::D;
  constexpr int PARTS = kCombineThreads / D;
  __shared__ float sw[kMaxSplits];
  __shared__ float sred[kCombineThreads];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int S = a.n_splits;
  const float* p = a.part + (int64_t)bh * S * (D + 2);

  float mx = kNegInf;
  for (int s = tid; s < S; s += kCombineThreads) mx = fmaxf(mx, p[(int64_t)s * (D + 2)]);
  sred[tid] = mx;
  __syncthreads();
  for (int o = kCombineThreads / 2; o > 0; o >>= 1) {
    if (tid < o) sred[tid] = fmaxf(sred[tid], sred[tid + o]);
    __syncthreads();
  }
  const float M = sred[0];
  __syncthreads();
  float lp = 0.f;
  for (int s = tid; s < S; s += kCombineThreads) {
    const float* ps = p + (int64_t)s * (D + 2);
    const float w = exp2f_fast(ps[0] - M);
    sw[s] = w;
    lp = fmaf(ps[1], w, lp);
  }
  sred[tid] = lp;
  __syncthreads();
  for (int o = kCombineThreads / 2; o > 0; o >>= 1) {
    if (tid < o) sred[tid] += sred[tid + o];
    __syncthreads();
  }
  const float L = sred[0];
  __syncthreads();
  const int dd = tid % D, part = tid / D;
  float O = 0.f;
#pragma unroll 8
  for (int s = part; s < S; s += PARTS) O = fmaf(p[(int64_t)s * (D + 2) + 2 + dd], sw[s], O);
  sred[tid] = O;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) acc += sred[q * D + tid];
    const float r = acc / L;
    if constexpr (sizeof(T) == 2) {
      reinterpret_cast<uint16_t*>(a.out)[(int64_t)bh * D + tid] = (uint16_t)f32_to_bf16_bits(r);
    } else {
      reinterpret_cast<float*>(a.out)[(int64_t)bh * D + tid] = r;
    }
    if (tid == 0) {
      const float lse2 = M + log2f_fast(L);
      if (a.lse2) a.lse2[bh] = lse2;
      if (a.lse_out) a.lse_out[bh] = lse2 * kLn2;
    }
  }
}

// pooled[b,g,j] = sum over the G heads h of group g of 2^(s[b,h,j] - lse2[b,h]),
// plus the row's histogram of key bits 31..21 (the select kernel's first
// digit), counted in LDS and added to the row's global histogram.
template <int G>
__global__ __launch_bounds__(256) void k_decode_pool(const PoolDecodeArgs a) {
  __shared__ uint32_t sh[2048];
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  for (int i = tid; i < 2048; i += 256) sh[i] = 0u;
  __syncthreads();
  const int j = (blockIdx.x * 256 + tid) * 4;
  float lse[G];
  const float* sp[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int64_t bh = (int64_t)b * a.Hq + g * G + hh;
    lse[hh] = a.lse2[bh];
    sp[hh] = a.scores + bh * a.N;
  }
  float* out = a.pooled + ((int64_t)b * a.Hkv + g) * a.N;
  if (j < a.N) {
    if (j + 4 <= a.N && (a.N & 3) == 0) {
      float4 s4[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) s4[hh] = *reinterpret_cast<const float4*>(sp[hh] + j);
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

template <typename T, int G>
hipError_t launch_splitk_t(const DecodeArgs& a, bool gather, hipStream_t s) {
  if (a.n_splits > kMaxSplits || a.n_splits < 1) return hipErrorInvalidValue;
  dim3 grid(a.n_splits, a.Hkv, a.B);
  if (gather) {
    size_t lds = (size_t)a.keys_per_split * sizeof(int32_t);
    hipLaunchKernelGGL((k_decode_splitk<T, G, true, false>), grid, dim3(kThreads), lds, s, a);
  } else if (a.scores) {
    hipLaunchKernelGGL((k_decode_splitk<T, G, false, true>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_decode_splitk<T, G, false, false>), grid, dim3(kThreads), 0, s, a);
  }
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

}  // namespace

hipError_t launch_decode_splitk(const DecodeArgs& a, int dtype, bool gather, hipStream_t s) {
  return dtype == 1 ? launch_splitk_g<uint16_t>(a, gather, s) : launch_splitk_g<float>(a, gather, s);
}

hipError_t launch_decode_combine(const CombineArgs& a, int dtype, hipStream_t s) {
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(k_decode_combine<uint16_t>, dim3(a.BH), dim3(kCombineThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_decode_combine<float>, dim3(a.BH), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_pool(const PoolDecodeArgs& a, hipStream_t s) {
  dim3 grid((a.N + 1023) / 1024, a.Hkv, a.B);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL(k_decode_pool<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_decode_pool<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_decode_pool<4>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_decode_pool<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kc
