// Exact Top-k selection over fp32 rows: radix select on order-preserving
// uint32 keys, then an index-ordered compaction.
//
// Method: anchors compute the EXACT Top-k key indices of the pooled
// post-softmax scores ([Abstract]; page "論文解説: Kascade …", section
// "アンカーレイヤーと再利用レイヤー").  Ties go to the lower index; the list is
// written in ascending index order.
//
// One workgroup (1024 threads, 16 waves) per row.
//   digit 0 (key bits 31..21): a 2048-bin histogram, either handed in (the
//     decode pooling kernel builds it while it writes the row) or counted
//     here;
//   digit 1 (bits 20..10): one sweep counts the keys whose digit 0 matches
//     and appends them to an LDS candidate buffer (wave-aggregated slots);
//   digit 2 (bits 9..0): counted over the candidates only (a full sweep if
//     the buffer overflowed).
// Each digit's bin is found with a block prefix sum from the top, which fixes
// the k-th largest key T exactly and how many keys equal to T are taken (the
// lowest-index ones).  The compaction walks the row in index order in tiles
// of 32768 keys (32 contiguous keys per thread) with a block prefix sum of
// (greater, equal) counts, so the output is ascending and deterministic.
// Histograms are integer LDS atomics: order-independent.  Rows up to the
// cache capacity are held in LDS as keys (one HBM read per row).
#include "common.h"
#include "kernels.h"
#include "radix.h"

namespace kc {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 2048;
constexpr int kRun = 32;          // contiguous keys per thread in a compaction tile
constexpr int kTileKeys = kSelThreads * kRun;
constexpr int kCandCap = 4096;    // digit-2 candidates kept in LDS

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
  const uint32_t incl = wave_incl_scan(x);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (tid < 64) {   // the whole first wave: its lanes past kSelWaves scan zeros
    const uint32_t w = tid < kSelWaves ? sh[tid] : 0u;
    const uint32_t wi = wave_incl_scan(w);
    if (tid < kSelWaves) sh[tid] = wi - w;          // exclusive wave offsets
    if (tid == kSelWaves - 1) sh[kSelWaves] = wi;   // block total
  }
  __syncthreads();
  const uint32_t r = sh[wave] + incl - x;
  total = sh[kSelWaves];
  __syncthreads();
  return r;
}

// Given a histogram (nb bins) of the keys still in play, find the bin that
// holds the need-th largest key.  Returns the bin; `above_out` receives the
// count of keys in higher bins.  Thread tid owns bins 2*rev+1 and 2*rev,
// rev = 1023 - tid, so the prefix sum runs from the top bin down.
KC_INLINE uint32_t find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* scan,
                            uint32_t* s_sel, uint32_t& above_out) {
  const int tid = threadIdx.x;
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
  const uint32_t bin = s_sel[0];
  above_out = s_sel[1];
  __syncthreads();
  return bin;
}

// Sweep the row's keys: 4 keys per step per thread (16-byte LDS reads when
// cached, 16-byte global loads when the row is aligned), f(j, key) per key.
template <typename F>
KC_INLINE void sweep(const RowGeom& g, const uint32_t* cache, bool cached, F&& f) {
  const int tid = threadIdx.x, n = g.n;
  const bool vec = cached || ((reinterpret_cast<uintptr_t>(g.src) & 15) == 0);
  const int nv = vec ? (n & ~3) : 0;
  constexpr int kB = 4;   // 16-byte loads in flight per thread
  for (int base = 0; base < nv; base += kSelThreads * 4 * kB) {
    uint4 w[kB];
#pragma unroll
    for (int e = 0; e < kB; ++e) {
      const int j = base + (e * kSelThreads + tid) * 4;
      w[e] = make_uint4(0, 0, 0, 0);
      if (j < nv) {
        if (cached) {
          w[e] = *reinterpret_cast<const uint4*>(cache + j);
        } else {
          const float4 v = *reinterpret_cast<const float4*>(g.src + j);
          w[e] = make_uint4(f32_order_key(v.x), f32_order_key(v.y), f32_order_key(v.z),
                            f32_order_key(v.w));
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kB; ++e) {
      const int j = base + (e * kSelThreads + tid) * 4;
      const bool in = j < nv;
      f(in, w[e].x);
      f(in, w[e].y);
      f(in, w[e].z);
      f(in, w[e].w);
    }
  }
  // tail (and unaligned rows): whole waves step together so ballots stay uniform
  for (int j0 = nv; j0 < n; j0 += kSelThreads) {
    const int j = j0 + tid;
    const bool in = j < n;
    f(in, in ? (cached ? cache[j] : f32_order_key(g.src[j])) : 0u);
  }
}

__global__ __launch_bounds__(kSelThreads) void k_topk_select(const SelectArgs a) {
  extern __shared__ __align__(16) uint32_t smem[];
  uint32_t* hist = smem;                       // kHistBins
  uint32_t* scan = smem + kHistBins;           // 32 words
  uint32_t* cand = smem + kHistBins + 32;      // kCandCap candidate keys
  uint32_t* cache = cand + kCandCap;           // row keys when cached
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_ncand;

  const RowGeom g = row_geom(a, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
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
  const uint32_t* hist0 = a.hist0 ? a.hist0 + (int64_t)blockIdx.x * kHistBins : nullptr;
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = hist0 ? hist0[i] : 0u;
  if (tid == 0) s_ncand = 0;
  if (cached) {
    // one pass over HBM: keys into LDS (16-byte loads when the row is aligned)
    const bool vec = (reinterpret_cast<uintptr_t>(g.src) & 15) == 0;
    const int nv = vec ? (n & ~3) : 0;
    for (int base = 0; base < nv; base += kSelThreads * 16) {
      float4 v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = base + (e * kSelThreads + tid) * 4;
        v[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nv) v[e] = *reinterpret_cast<const float4*>(g.src + j);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = base + (e * kSelThreads + tid) * 4;
        if (j < nv)
          *reinterpret_cast<uint4*>(cache + j) = make_uint4(
              f32_order_key(v[e].x), f32_order_key(v[e].y), f32_order_key(v[e].z),
              f32_order_key(v[e].w));
      }
    }
    for (int j = nv + tid; j < n; j += kSelThreads) cache[j] = f32_order_key(g.src[j]);
  }
  __syncthreads();

  // digit 0
  if (!hist0) {
    sweep(g, cache, cached, [&](bool in, uint32_t key) {
      if (in) atomicAdd(&hist[key >> 21], 1u);
    });
    __syncthreads();
  }
  uint32_t need = (uint32_t)k, above;
  const uint32_t b0 = find_bin(hist, 2048, need, scan, s_sel, above);
  need -= above;

  // digit 1, collecting the digit-0 matches as candidates
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  sweep(g, cache, cached, [&](bool in, uint32_t key) {
    const bool m = in && (key >> 21) == b0;
    if (m) atomicAdd(&hist[(key >> 10) & 2047u], 1u);
    const uint64_t bal = __ballot(m);
    if (bal) {
      uint32_t base = 0;
      const int leader = __ffsll((unsigned long long)bal) - 1;
      if (lane == leader) base = atomicAdd(&s_ncand, (uint32_t)__popcll(bal));
      base = __shfl(base, leader, 64);
      const uint32_t slot = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
      if (m && slot < (uint32_t)kCandCap) cand[slot] = key;
    }
  });
  __syncthreads();
  const uint32_t b1 = find_bin(hist, 2048, need, scan, s_sel, above);
  need -= above;
  const uint32_t p01 = (b0 << 11) | b1;   // bits 31..10 of T

  // digit 2
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  const uint32_t ncand = s_ncand;
  if (ncand <= (uint32_t)kCandCap) {
    for (uint32_t i = tid; i < ncand; i += kSelThreads) {
      const uint32_t key = cand[i];
      if ((key >> 10) == p01) atomicAdd(&hist[key & 1023u], 1u);
    }
  } else {
    sweep(g, cache, cached, [&](bool in, uint32_t key) {
      if (in && (key >> 10) == p01) atomicAdd(&hist[key & 1023u], 1u);
    });
  }
  __syncthreads();
  const uint32_t b2 = find_bin(hist, 1024, need, scan, s_sel, above);
  need -= above;
  const uint32_t T = (p01 << 10) | b2;   // the k-th largest key; take `need` of the keys == T

  // compaction in index order
  const bool vec = cached || ((reinterpret_cast<uintptr_t>(g.src) & 15) == 0);
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += kTileKeys) {
    const int j0 = base + tid * kRun;
    uint32_t keys[kRun];
#pragma unroll
    for (int e = 0; e < kRun; e += 4) {
      const int j = j0 + e;
      if (vec && j + 4 <= n) {
        uint4 w;
        if (cached) {
          w = *reinterpret_cast<const uint4*>(cache + j);
        } else {
          const float4 v = *reinterpret_cast<const float4*>(g.src + j);
          w = make_uint4(f32_order_key(v.x), f32_order_key(v.y), f32_order_key(v.z),
                         f32_order_key(v.w));
        }
        keys[e] = w.x; keys[e + 1] = w.y; keys[e + 2] = w.z; keys[e + 3] = w.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          keys[e + q] = (j + q < n) ? (cached ? cache[j + q] : f32_order_key(g.src[j + q])) : 0u;
      }
    }
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      const bool in = j0 + e < n;
      cgt += (in && keys[e] > T) ? 1u : 0u;
      ceq += (in && keys[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((cgt << 16) | ceq, scan, tot);
    uint32_t gt = run_gt + (ex >> 16), eq = run_eq + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      const int j = j0 + e;
      if (j < n) {
        if (keys[e] > T) {
          g.out[gt + min(eq, need)] = j;
          ++gt;
        } else if (keys[e] == T) {
          if (eq < need) g.out[gt + eq] = j;
          ++eq;
        }
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
  for (int j = k + tid; j < g.out_len; j += kSelThreads) g.out[j] = -1;
}

}  // namespace

// LDS bytes of the select kernel for a given row cache capacity.
// ---- wide select: few long rows, many workgroups per row ------------------
//
// The same radix select (digits of 11, 11 and 10 bits) and index-ordered
// compaction as k_topk_select, spread over chunks of CH keys (wide_chunk(n)),
// in two passes after the pooling pass that built digit 0's histogram:
//   pass A (chunks x rows): every chunk finds digit 0's bin b0 from the
//     complete histogram, counts its keys above b0 (all selected), and
//     histograms digit 1 of its keys in b0 (the candidates: LDS, then integer
//     atomics into hist1) and stores them in index order at its own offset
//     of the row's candidate buffer;
//   pass B (chunks x rows): every chunk resolves digits 1 and 2 (digit 2 over
//     the row's candidates), which fixes the k-th largest key T and how many
//     keys equal to T are taken, counts the keys > T and == T of the chunks
//     before it (their keys above b0 plus their candidates compared with T),
//     and writes its own selected indices in index order.
// Every workgroup repeats the small histogram scans instead of waiting for
// another; the kernel boundary orders the passes.  Histograms are integer
// atomics and candidates sit at fixed per-chunk offsets, so the output is
// deterministic.  (A third pass that summed per-chunk counts written by pass
// B measured 1.5 us slower per 32K anchor layer.)

// The thread's CH/256 consecutive keys of chunk c (keys past n read as 0;
// every use checks the position against n).
template <int CH, int PT = CH / kWideThreads>
KC_INLINE void chunk_keys(const WideSelectArgs& a, const float* src, int c, uint32_t (&key)[PT], int& j0) {
  static_assert(PT % 4 == 0, "whole 16-byte loads");
  constexpr int kPerThread = PT;
  j0 = c * CH + threadIdx.x * kPerThread;
  const bool vec = (a.row_stride & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.src) & 15) == 0);
  if (vec && j0 + kPerThread <= a.n) {
#pragma unroll
    for (int q = 0; q < kPerThread; q += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + j0 + q);
      key[q] = f32_order_key(v.x);
      key[q + 1] = f32_order_key(v.y);
      key[q + 2] = f32_order_key(v.z);
      key[q + 3] = f32_order_key(v.w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) key[q] = j0 + q < a.n ? f32_order_key(src[j0 + q]) : 0u;
  }
}

// Pass A (chunks x rows): digit 0's bin b0 from the complete histogram; the
// chunk's keys above b0 are counted (all selected), its keys in b0 (the
// candidates) are counted, histogrammed on digit 1 (LDS, then integer atomics
// into hist1) and stored in index order at the chunk's own offset of the
// row's candidate buffer.  chunk_cnt[row][c] = {keys above b0, candidates}.
template <int CH>
__global__ __launch_bounds__(kWideThreads) void k_select_wide_a(const WideSelectArgs a) {
  constexpr int kPerThread = CH / kWideThreads;
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t sh[8], s_sel[2];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const float* src = a.src + (int64_t)row * a.row_stride;
  // the histogram's bins and the chunk's keys are independent: both loads go
  // out before either is used
  uint32_t h0[kHistBins / kWideThreads];
  load_bins<kHistBins>(a.hist0 + (int64_t)row * kHistBins, h0);
  uint32_t key[kPerThread];
  int j0;
  chunk_keys<CH>(a, src, c, key, j0);
  uint32_t above;
  const uint32_t b0 = find_bin256_regs<kHistBins>(h0, (uint32_t)a.k, sh, s_sel, above);
  for (int i = tid; i < kHistBins; i += kWideThreads) hist[i] = 0u;
  __syncthreads();
  uint32_t cnt = 0, hi = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const bool in = j0 + q < a.n;
    const uint32_t d0 = key[q] >> 21;
    const bool m = in && d0 == b0;
    if (m) atomicAdd(&hist[(key[q] >> 10) & 2047u], 1u);
    cnt += m ? 1u : 0u;
    hi += (in && d0 > b0) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t off = scan256((cnt << 16) | hi, sh, tot);
  uint32_t* cand = a.cand + (int64_t)row * a.n + (int64_t)c * CH + (off >> 16);
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    if (j0 + q < a.n && (key[q] >> 21) == b0) *cand++ = key[q];
  }
  if (tid == 0) {
    uint32_t* cc = a.chunk_cnt + ((int64_t)row * a.chunks + c) * 2;
    cc[0] = tot & 0xFFFFu;
    cc[1] = tot >> 16;
  }
  uint32_t* h1 = a.hist1 + (int64_t)row * kHistBins;
  for (int i = tid; i < kHistBins; i += kWideThreads) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(h1 + i, v);
  }
}

// Candidate f of the row in chunk order: its chunk (by binary search over the
// exclusive prefix `cpre` of the chunks' candidate counts) and its key.
KC_INLINE uint32_t flat_cand(const WideSelectArgs& a, int row, int CH, const uint32_t* cpre, int chunks,
                             uint32_t f, int& cc) {
  int lo = 0, hi = chunks - 1;   // last chunk whose prefix is <= f
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cpre[mid] <= f) lo = mid;
    else hi = mid - 1;
  }
  cc = lo;
  return a.cand[(int64_t)row * a.n + (int64_t)lo * CH + (f - cpre[lo])];
}

// Pass B (chunks x rows): every chunk resolves digits 1 and 2 (digit 2 over
// the row's candidates), which fixes the k-th largest key T and how many keys
// equal to T are taken; it counts the keys > T and == T of the chunks before
// it (their keys above b0 plus their candidates compared with T) and writes
// its own selected indices in index order.
template <int CH>
__global__ __launch_bounds__(kWideThreads) void k_select_wide_b(const WideSelectArgs a) {
  constexpr int kPerThread = CH / kWideThreads;
  constexpr int kMaxCh = 1024;   // chunks per row on this path
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t cpre[kMaxCh];
  __shared__ uint32_t sh[8], s_sel[2];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int chunks = a.chunks;
  const float* src = a.src + (int64_t)row * a.row_stride;
  // independent loads first, all in flight together: both histograms' bins,
  // the chunks' counts (keys above b0 of the chunks before this one, and the
  // candidate counts for the flattened candidate index) and the chunk's keys
  uint32_t h0[kHistBins / kWideThreads], h1[kHistBins / kWideThreads];
  load_bins<kHistBins>(a.hist0 + (int64_t)row * kHistBins, h0);
  load_bins<kHistBins>(a.hist1 + (int64_t)row * kHistBins, h1);
  const uint32_t* ccnt = a.chunk_cnt + (int64_t)row * chunks * 2;
  uint32_t nc[kMaxCh / kWideThreads], abv = 0, csum = 0;
#pragma unroll
  for (int u = 0; u < kMaxCh / kWideThreads; ++u) {
    const int i = tid * (kMaxCh / kWideThreads) + u;
    nc[u] = i < chunks ? ccnt[2 * i + 1] : 0u;
    abv += (i < chunks && i < c) ? ccnt[2 * i] : 0u;
    csum += nc[u];
  }
  uint32_t key[kPerThread];
  int j0;
  chunk_keys<CH>(a, src, c, key, j0);
  uint32_t need = (uint32_t)a.k, above;
  const uint32_t b0 = find_bin256_regs<kHistBins>(h0, need, sh, s_sel, above);
  need -= above;
  const uint32_t b1 = find_bin256_regs<kHistBins>(h1, need, sh, s_sel, above);
  need -= above;
  const uint32_t p01 = (b0 << 11) | b1;
  // the candidate counts' prefix, and the block total of the keys above b0
  // in the chunks before chunk c
  uint32_t run, abv_ex, ncand, above_before;
  scan256x2(csum, abv, sh, run, abv_ex, ncand, above_before);
#pragma unroll
  for (int u = 0; u < kMaxCh / kWideThreads; ++u) {
    const int i = tid * (kMaxCh / kWideThreads) + u;
    if (i < kMaxCh) cpre[i] = run;
    run += nc[u];
  }
  for (int i = tid; i < 1024; i += kWideThreads) hist[i] = 0u;
  __syncthreads();   // cpre and the cleared histogram
  for (uint32_t f = tid; f < ncand; f += kWideThreads) {
    int cc;
    const uint32_t key = flat_cand(a, row, CH, cpre, chunks, f, cc);
    if ((key >> 10) == p01) atomicAdd(&hist[key & 1023u], 1u);
  }
  __syncthreads();
  const uint32_t b2 = find_bin256<1024>(hist, need, sh, s_sel, above);
  need -= above;
  const uint32_t T = (p01 << 10) | b2;   // the k-th largest key; `need` keys == T are taken
  // candidates of the chunks before this one: > T and == T
  const uint32_t fend = c < chunks ? cpre[c] : ncand;
  uint32_t gtc = 0, eqc = 0;
  for (uint32_t f = tid; f < fend; f += kWideThreads) {
    int cc;
    const uint32_t key = flat_cand(a, row, CH, cpre, chunks, f, cc);
    gtc += key > T ? 1u : 0u;
    eqc += key == T ? 1u : 0u;
  }
  uint32_t gtc_ex, eqc_ex, gt_before, eq_before;
  scan256x2(gtc, eqc, sh, gtc_ex, eqc_ex, gt_before, eq_before);   // block totals
  gt_before += above_before;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const bool in = j0 + q < a.n;
    gt += (in && key[q] > T) ? 1u : 0u;
    eq += (in && key[q] == T) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = scan256((gt << 16) | eq, sh, tot);
  uint32_t g2 = gt_before + (ex >> 16), e2 = eq_before + (ex & 0xFFFFu);
  int32_t* out = a.idx + (int64_t)row * a.idx_stride;
  const uint32_t kk = (uint32_t)a.k;   // positions stay inside the row's k slots
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int j = j0 + q;
    if (j < a.n) {
      if (key[q] > T) {
        const uint32_t pos = g2 + min(e2, need);
        if (pos < kk) out[pos] = j;
        ++g2;
      } else if (key[q] == T) {
        if (e2 < need && g2 + e2 < kk) out[g2 + e2] = j;
        ++e2;
      }
    }
  }
}

template <int CH>
hipError_t launch_wide_ch(const WideSelectArgs& a, hipStream_t s) {
  const dim3 grid(a.chunks, a.rows);
  hipLaunchKernelGGL(k_select_wide_a<CH>, grid, dim3(kWideThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select_wide_b<CH>, grid, dim3(kWideThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_select_wide(const WideSelectArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int ch = wide_chunk(a.n);
  if (a.chunks != (a.n + ch - 1) / ch || a.chunks > 1024) return hipErrorInvalidValue;
  return ch == kWideChunkShort ? launch_wide_ch<kWideChunkShort>(a, s) : launch_wide_ch<kWideChunk>(a, s);
}

size_t topk_select_lds_bytes(int cache_cap) {
  return (size_t)(kHistBins + 32 + kCandCap + cache_cap) * sizeof(uint32_t);
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
