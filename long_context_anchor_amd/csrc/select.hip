// Exact Top-k selection over fp32 rows: radix select on order-preserving
// uint32 keys, then an index-ordered compaction.
//
// Method: anchors compute the EXACT Top-k key indices of the pooled
// post-softmax scores ([Abstract]; page "論文解説: Kascade …", section
// "アンカーレイヤーと再利用レイヤー").  Ties go to the lower index; the list is
// written in ascending index order.
//
// One workgroup (1024 threads, 16 waves) per row.  Three histogram passes
// over 11/11/10-bit digits (MSB first) fix the k-th largest key T exactly and
// how many elements equal to T are taken (the lowest-index ones).  A final
// pass in index order writes every key > T and the first `need` keys == T,
// using block prefix sums, so the output is ascending and deterministic.  The
// histograms are integer LDS atomics: order-independent.  Rows that fit are
// cached as keys in LDS so the four passes read the row from HBM once.
#include "common.h"
#include "kernels.h"

namespace kc {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 2048;
constexpr int kRun = 8;   // contiguous elements per thread in the compaction pass
constexpr int kBatch = 8; // independent loads in flight per thread in the scans

struct RowGeom {
  const float* src;
  int32_t n, k;
  int32_t* out;
  int32_t out_len;   // k padded with -1 up to out_len
};

KC_INLINE RowGeom row_geom(const SelectArgs& a, int r) {
  RowGeom g;
  if (a.mode == 0) {
    g.src = a.src + (int64_t)r * a.row_stride;
    g.n = a.n;
    g.k = min(a.k, a.n);
    g.out = a.idx + (int64_t)r * a.idx_stride;
    g.out_len = g.k;
  } else {
    // r enumerates (b, t, g) with g fastest
    const int gg = r % a.Hkv;
    const int t = (r / a.Hkv) % a.T;
    const int b = r / (a.Hkv * a.T);
    const int P = min(a.N, a.tile * (t + 1));
    g.src = a.src + (int64_t)b * a.packed_per_batch + packed_row_offset(t, gg, a.Hkv, a.tile, a.N);
    g.n = P;
    g.k = tile_k_for_len(P, a.pct, a.round_to, a.k_min);
    g.out = a.idx + ((int64_t)(b * a.T + t) * a.Hkv + gg) * a.idx_stride;
    g.out_len = (int32_t)a.idx_stride;
  }
  return g;
}

// Exclusive prefix sum over the block (1024 threads).  `sh` holds >= 17 words.
KC_INLINE uint32_t block_excl_scan(uint32_t x, uint32_t* sh, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (tid < 64) {
    uint32_t w = tid < kSelWaves ? sh[tid] : 0u;
    uint32_t wi = w;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      uint32_t y = __shfl_up(wi, o, 64);
      if (lane >= o) wi += y;
    }
    if (tid < kSelWaves) sh[tid] = wi - w;          // exclusive wave offsets
    if (tid == kSelWaves - 1) sh[kSelWaves] = wi;   // block total
  }
  __syncthreads();
  const uint32_t r = sh[wave] + incl - x;
  total = sh[kSelWaves];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kSelThreads) void k_topk_select(const SelectArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;                       // kHistBins
  uint32_t* scan = smem + kHistBins;           // 32 words
  uint32_t* cache = smem + kHistBins + 32;     // row keys when cached
  __shared__ uint32_t s_sel[2];

  const RowGeom g = row_geom(a, blockIdx.x);
  const int tid = threadIdx.x;
  const int n = g.n, k = g.k;

  if (k >= n) {   // every index is selected
    for (int j = tid; j < g.out_len; j += kSelThreads) g.out[j] = j < n ? j : -1;
    return;
  }
  if (k <= 0) {
    for (int j = tid; j < g.out_len; j += kSelThreads) g.out[j] = -1;
    return;
  }
  const bool cached = n <= a.cache_cap;
  if (cached) {
    // kBatch independent loads in flight per thread
    for (int base = 0; base < n; base += kSelThreads * kBatch) {
      float v[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const int j = base + e * kSelThreads + tid;
        v[e] = j < n ? g.src[j] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const int j = base + e * kSelThreads + tid;
        if (j < n) cache[j] = f32_order_key(v[e]);
      }
    }
  }

  uint32_t prefix = 0;
  uint32_t need = (uint32_t)k;   // how many still to take among keys matching prefix
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int nbits = pass == 2 ? 10 : 11;
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = 1 << nbits;
    const int hs = sh + nbits;                 // bits above this digit
    for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kSelThreads * kBatch) {
      uint32_t kk[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const int j = base + e * kSelThreads + tid;
        kk[e] = j < n ? (cached ? cache[j] : f32_order_key(g.src[j])) : 0u;
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const int j = base + e * kSelThreads + tid;
        const bool match = j < n && ((pass == 0) || ((kk[e] >> hs) == prefix));
        if (match) atomicAdd(&hist[(kk[e] >> sh) & (nb - 1)], 1u);
      }
    }
    __syncthreads();
    // thread tid owns bins (from the top) 2*tid and 2*tid+1 of the reversed order
    const int rev = kSelThreads - 1 - tid;
    const int bh = 2 * rev + 1, bl = 2 * rev;
    const uint32_t ch = bh < nb ? hist[bh] : 0u;
    const uint32_t cl = bl < nb ? hist[bl] : 0u;
    uint32_t total;
    const uint32_t above = block_excl_scan(ch + cl, scan, total);
    if (bh < nb && above < need && above + ch >= need) {
      s_sel[0] = (uint32_t)bh;
      s_sel[1] = above;
    } else if (bl < nb && above + ch < need && above + ch + cl >= need) {
      s_sel[0] = (uint32_t)bl;
      s_sel[1] = above + ch;
    }
    __syncthreads();
    prefix = (prefix << nbits) | s_sel[0];
    need -= s_sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;   // the k-th largest key; take `need` of the keys == T

  // compaction in index order
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += kSelThreads * kRun) {
    const int j0 = base + tid * kRun;
    uint32_t keys[kRun];
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      const int j = j0 + e;
      uint32_t key = 0;
      if (j < n) key = cached ? cache[j] : f32_order_key(g.src[j]);
      keys[e] = key;
      cgt += (j < n && key > T) ? 1u : 0u;
      ceq += (j < n && key == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((cgt << 16) | ceq, scan, tot);
    uint32_t gt = run_gt + (ex >> 16), eq = run_eq + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      const int j = j0 + e;
      if (j >= n) break;
      if (keys[e] > T) {
        g.out[gt + min(eq, need)] = j;
        ++gt;
      } else if (keys[e] == T) {
        if (eq < need) g.out[gt + eq] = j;
        ++eq;
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
  for (int j = k + tid; j < g.out_len; j += kSelThreads) g.out[j] = -1;
}

}  // namespace

// LDS bytes of the select kernel for a given row cache capacity.
size_t topk_select_lds_bytes(int cache_cap) {
  return (size_t)(kHistBins + 32 + cache_cap) * sizeof(uint32_t);
}

hipError_t topk_select_set_max_lds(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_topk_select),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_topk_select(const SelectArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_select, dim3(a.rows), dim3(kSelThreads),
                     topk_select_lds_bytes(a.cache_cap), s, a);
  return hipGetLastError();
}

}  // namespace kc
