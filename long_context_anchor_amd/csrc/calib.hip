// Calibration: per-KV-head cross-layer similarity of pooled attention rows,
// the layer weight, and the host-side steps that turn them into an anchor
// set and head maps.
//
// Method (page "論文解説: Kascade …"): eq. sim of section
// "レイヤー間類似度とアンカーレイヤー選択" compares layer b's distribution on layer
// a's Top-k set with its mass on its own Top-k set; section "ヘッドリマッピング"
// pairs every KV head of a reuse layer with the most similar KV head of its
// anchor; eq. w weights a layer by 1 - cos(input, output); the DP of section
// "動的計画法（Algorithm 1）" picks the anchors that maximise the weighted
// similarity they cover.
//
// The pooled rows and Top-k lists come from the anchor decode pass run on
// every layer (its pooled_out and topk_idx), so the GPU part is one gather
// reduction: for every pair of layers a <= b, heads (ga, gb) and sample s,
// the sum of pooled_b[s, gb] over list_a[s, ga].  Sums are fp64 in a fixed
// order (no atomics): results are deterministic.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace kc {

namespace {

constexpr int kCalThreads = 256;

// Sum over the workgroup, fp64, fixed order.
KC_INLINE double block_sum_f64(double x, double* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kCalThreads / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Sum of row[list[i]], i < k (positions clamped into the row).
KC_INLINE double gather_sum(const float* row, const int32_t* list, int k, int n, double* red) {
  double s = 0.0;
  for (int i = threadIdx.x; i < k; i += kCalThreads) {
    const int j = min(max(list[i], 0), n - 1);
    s += (double)row[j];
  }
  return block_sum_f64(s, red);
}

// One workgroup per (gb, layer b, layer a); pairs with a > b exit.
__global__ __launch_bounds__(kCalThreads) void k_calib_sim(const float* __restrict__ pooled,
                                                          const int32_t* __restrict__ idx, int L,
                                                          int S, int Hkv, int N, int k,
                                                          float* __restrict__ sim) {
  const int gb = blockIdx.x, lb = blockIdx.y, la = blockIdx.z;
  if (la > lb) return;
  __shared__ double red[kCalThreads / 64];
  __shared__ double acc[kMaxKvHeads];
  const int tid = threadIdx.x;
  for (int ga = tid; ga < Hkv; ga += kCalThreads) acc[ga] = 0.0;
  __syncthreads();
  for (int s = 0; s < S; ++s) {
    const float* pb = pooled + (((int64_t)lb * S + s) * Hkv + gb) * N;
    const int32_t* ib = idx + (((int64_t)lb * S + s) * Hkv + gb) * k;
    const double norm = gather_sum(pb, ib, k, N, red);
    for (int ga = 0; ga < Hkv; ++ga) {
      const int32_t* ia = idx + (((int64_t)la * S + s) * Hkv + ga) * k;
      const double m = gather_sum(pb, ia, k, N, red);
      if (tid == 0) acc[ga] += norm > 0.0 ? m / norm : 0.0;
    }
  }
  __syncthreads();
  for (int ga = tid; ga < Hkv; ga += kCalThreads)
    sim[(((int64_t)la * L + lb) * Hkv + ga) * Hkv + gb] = (float)(acc[ga] / S);
}

// Per-token cosine of x and y (rows of `dim` elements), partial sums per
// workgroup of 64 tokens; a token with a zero vector makes its cosine NaN.
template <typename T>
__global__ __launch_bounds__(kCalThreads) void k_cosine_partial(const T* __restrict__ x,
                                                               const T* __restrict__ y, int tokens,
                                                               int dim, double* __restrict__ part) {
  __shared__ double red[kCalThreads / 64];
  __shared__ double cs[64];
  const int t0 = blockIdx.x * 64, tid = threadIdx.x;
  for (int tt = 0; tt < 64; ++tt) {
    const int t = t0 + tt;
    double xy = 0.0, xx = 0.0, yy = 0.0;
    if (t < tokens) {
      for (int i = tid; i < dim; i += kCalThreads) {
        double xv, yv;
        if constexpr (std::is_same<T, _Float16>::value) {
          xv = (double)x[(int64_t)t * dim + i];
          yv = (double)y[(int64_t)t * dim + i];
        } else if constexpr (sizeof(T) == 2) {
          xv = (double)bf16_lo((uint32_t)x[(int64_t)t * dim + i]);
          yv = (double)bf16_lo((uint32_t)y[(int64_t)t * dim + i]);
        } else {
          xv = (double)x[(int64_t)t * dim + i];
          yv = (double)y[(int64_t)t * dim + i];
        }
        xy += xv * yv;
        xx += xv * xv;
        yy += yv * yv;
      }
    }
    xy = block_sum_f64(xy, red);
    xx = block_sum_f64(xx, red);
    yy = block_sum_f64(yy, red);
    if (tid == 0) cs[tt] = t < tokens ? xy / (sqrt(xx) * sqrt(yy)) : 0.0;
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int tt = 0; tt < 64; ++tt) s += cs[tt];
    part[blockIdx.x] = s;
  }
}

// w = 1 - mean cosine, summing the partials in order.
__global__ __launch_bounds__(64) void k_cosine_final(const double* __restrict__ part, int nparts,
                                                    int tokens, float* __restrict__ w) {
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < nparts; ++i) s += part[i];
    *w = (float)(1.0 - s / tokens);
  }
}

}  // namespace

hipError_t launch_calib_sim(const float* pooled, const int32_t* idx, int L, int S, int Hkv, int N,
                            int k, float* sim, hipStream_t s) {
  hipLaunchKernelGGL(k_calib_sim, dim3(Hkv, L, L), dim3(kCalThreads), 0, s, pooled, idx, L, S, Hkv,
                     N, k, sim);
  return hipGetLastError();
}

hipError_t launch_layer_weight(const void* x, const void* y, int tokens, int dim, int dtype,
                               double* part, float* w, hipStream_t s) {
  const int nparts = (tokens + 63) / 64;
  if (dtype == 2)
    hipLaunchKernelGGL(k_cosine_partial<_Float16>, dim3(nparts), dim3(kCalThreads), 0, s,
                       reinterpret_cast<const _Float16*>(x), reinterpret_cast<const _Float16*>(y),
                       tokens, dim, part);
  else if (dtype == 1)
    hipLaunchKernelGGL(k_cosine_partial<uint16_t>, dim3(nparts), dim3(kCalThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(y),
                       tokens, dim, part);
  else
    hipLaunchKernelGGL(k_cosine_partial<float>, dim3(nparts), dim3(kCalThreads), 0, s,
                       reinterpret_cast<const float*>(x), reinterpret_cast<const float*>(y), tokens,
                       dim, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_cosine_final, dim3(1), dim3(64), 0, s, part, nparts, tokens, w);
  return hipGetLastError();
}

}  // namespace kc
