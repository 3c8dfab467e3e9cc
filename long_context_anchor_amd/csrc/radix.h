// Block-wide radix helpers of the exact Top-k selection (256-thread
// workgroups): an exclusive prefix sum and the histogram bin that holds the
// need-th largest key, scanning from the top bin down.
#pragma once
#include "common.h"

namespace kc {

constexpr int kWideThreads = 256;
constexpr int kWideWaves = kWideThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wave (every lane active) with
// DPP moves instead of LDS shuffles: shifts by 1, 2, 4 and 8 lanes inside
// each 16-lane row (a lane with no source adds nothing), then lane 15 of
// rows 0 and 2 added to rows 1 and 3, then lane 31 added to rows 2 and 3.
KC_INLINE uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the 256-thread block; `sh` holds >= 5 words.
// TAIL = false leaves out the closing barrier: the caller then puts a block
// barrier between this call and the next write of `sh`.
template <bool TAIL = true>
KC_INLINE uint32_t scan256(uint32_t x, uint32_t* sh, uint32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_incl_scan(x);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWideWaves; ++w) {
    const uint32_t v = sh[w];
    before += w < wave ? v : 0u;
    tot += v;
  }
  if (TAIL) __syncthreads();
  total = tot;
  return before + incl - x;
}

// Two independent exclusive prefix sums over the block behind one pair of
// barriers; `sh` holds >= 8 words.
KC_INLINE void scan256x2(uint32_t x, uint32_t y, uint32_t* sh, uint32_t& ex, uint32_t& ey,
                         uint32_t& tx, uint32_t& ty) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ix = wave_incl_scan(x), iy = wave_incl_scan(y);
  if (lane == 63) {
    sh[wave] = ix;
    sh[kWideWaves + wave] = iy;
  }
  __syncthreads();
  uint32_t bx = 0, by = 0, sx = 0, sy = 0;
#pragma unroll
  for (int w = 0; w < kWideWaves; ++w) {
    const uint32_t vx = sh[w], vy = sh[kWideWaves + w];
    bx += w < wave ? vx : 0u;
    by += w < wave ? vy : 0u;
    sx += vx;
    sy += vy;
  }
  __syncthreads();
  ex = bx + ix - x;
  ey = by + iy - y;
  tx = sx;
  ty = sy;
}

// Bin of a histogram (nb = 2048 or 1024 bins, global or LDS) holding the
// need-th largest key, scanning from the top bin down; `above` receives the
// count of keys in higher bins.  Two block barriers; the histogram (when in
// LDS) and `sh` may be rewritten after the call, `s_sel` only behind a later
// barrier.  Thread t owns nb/256 consecutive bins
// counted from the top: load_bins reads them (so a caller can issue the
// loads early, beside other independent ones), find_bin256_regs searches.
template <int NB>
KC_INLINE void load_bins(const uint32_t* hist, uint32_t (&h)[NB / kWideThreads]) {
  constexpr int W = NB / kWideThreads;
  const int hi = NB - W * (int)threadIdx.x;   // bins [hi - W, hi)
#pragma unroll
  for (int i = 0; i < W; ++i) h[i] = hist[hi - 1 - i];
}

template <int NB>
KC_INLINE uint32_t find_bin256_regs(const uint32_t (&h)[NB / kWideThreads], uint32_t need, uint32_t* sh,
                                    uint32_t* s_sel, uint32_t& above) {
  constexpr int W = NB / kWideThreads;
  const int tid = threadIdx.x;
  const int hi = NB - W * tid;
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) tot += h[i];
  uint32_t all;
  // the barrier below the search closes the scan: `sh` is read before it
  const uint32_t before = scan256<false>(tot, sh, all);
  // need = 0, or a histogram holding fewer than `need` keys: bin 0, nothing
  // above (no thread finds a bin); else exactly one thread finds it
  const bool none = need == 0u || all < need;
  if (!none && before < need && before + tot >= need) {
    uint32_t cum = before;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (cum + h[i] >= need) {
        s_sel[0] = (uint32_t)(hi - 1 - i);
        s_sel[1] = cum;
        break;
      }
      cum += h[i];
    }
  }
  __syncthreads();
  // No closing barrier: the next write of `s_sel` (by the next search's
  // finder) comes after that search's scan barrier, which every thread
  // reaches only after reading these two words here.
  above = none ? 0u : s_sel[1];
  return none ? 0u : s_sel[0];
}

template <int NB>
KC_INLINE uint32_t find_bin256(const uint32_t* hist, uint32_t need, uint32_t* sh, uint32_t* s_sel,
                               uint32_t& above) {
  uint32_t h[NB / kWideThreads];
  load_bins<NB>(hist, h);
  return find_bin256_regs<NB>(h, need, sh, s_sel, above);
}

}  // namespace kc
