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
  __syncthreads();
  total = tot;
  return before + incl - x;
}

// Bin of a histogram (nb = 2048 or 1024 bins, global or LDS) holding the
// need-th largest key, scanning from the top bin down; `above` receives the
// count of keys in higher bins.  Thread t owns nb/256 consecutive bins
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
  if (tid == 0) {   // a histogram holding fewer than `need` keys selects bin 0
    s_sel[0] = 0u;
    s_sel[1] = 0u;
  }
  uint32_t all;
  const uint32_t before = scan256(tot, sh, all);
  if (before < need && before + tot >= need) {
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
  const uint32_t bin = s_sel[0];
  above = s_sel[1];
  __syncthreads();
  return bin;
}

template <int NB>
KC_INLINE uint32_t find_bin256(const uint32_t* hist, uint32_t need, uint32_t* sh, uint32_t* s_sel,
                               uint32_t& above) {
  uint32_t h[NB / kWideThreads];
  load_bins<NB>(hist, h);
  return find_bin256_regs<NB>(h, need, sh, s_sel, above);
}

}  // namespace kc
