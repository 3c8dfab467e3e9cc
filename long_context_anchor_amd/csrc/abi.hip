// C ABI of libkascade: argument validation, workspace layout, launch
// sequencing and per-kernel event timing.  Every check happens before the
// first launch, so a rejected call leaves all outputs untouched.
#include <math.h>
#include <atomic>
#include <mutex>
#include <string.h>
#include <vector>

#include "../../include/kascade.h"
#include "kernels.h"

using namespace kc;

// stream.hip: the stream-read reference (a measurement helper, not part of
// the method, so it stays out of the kernels' shared header)
namespace kc {
hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, int grid, hipStream_t s);
}

namespace {

thread_local int g_last_hip_error = 0;


constexpr int kMaxDevices = 64;

// Scratch of the allocation-free reuse decode (kascade_reuse_decode_noalloc):
// split partials and per-head log2-lse live in this file-scope device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel: the device address comes from hipGetSymbolAddress
// (DeviceInfo::scratch, taken once per device at set-up).
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceInfo {
  bool init = false;
  void* scratch = nullptr;   // device address of this GPU's scratch array
  int select_cache_cap = 0;
  int cus = 0;
  size_t lds_per_cu = 0;
  // split-K variants [dtype][log2 G][kind] (kind 0 dense, 1 dense + score
  // spill, 2 gather; +3 for a paged cache): resident workgroups per CU
  // without dynamic LDS (0 = not queried yet) and static LDS bytes
  int splitk_bpc[3][4][6] = {};
  size_t splitk_lds[3][4][6] = {};
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

int device_setup(DeviceInfo** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KASCADE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return KASCADE_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.init) {
    int lds = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return KASCADE_ERR_HIP;
    }
    // select kernel: 2048-bin histogram + scan scratch + row cache
    int cap = (int)((lds - (int)topk_select_lds_bytes(0)) / 4);
    cap = cap > 32768 ? 32768 : cap;
    cap = cap < 0 ? 0 : (cap & ~1023);
    e = topk_select_set_max_lds(topk_select_lds_bytes(cap));
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return KASCADE_ERR_HIP;
    }
    d.select_cache_cap = cap;
    e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    int lds_cu = 0;
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess) e = decode_set_max_lds();
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return KASCADE_ERR_HIP;
    }
    d.lds_per_cu = (size_t)lds_cu;
    e = prefill_set_max_lds();
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return KASCADE_ERR_HIP;
    }
    // this device's copy of the scratch array (the device is current here)
    void* sp = nullptr;
    e = hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch));
    if (e != hipSuccess || sp == nullptr) {
      g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return KASCADE_ERR_HIP;
    }
    d.scratch = sp;
    d.init = true;
  }
  *out = &d;
  return KASCADE_OK;
}

// Workgroup slots of the whole GPU for one split-K variant running splits of
// kps keys: CUs x resident workgroups (registers or LDS, whichever binds).
int splitk_slots(DeviceInfo* d, int dtype, int G, bool gather, bool spill, bool paged, int kps,
                 int* slots) {
  const int lg = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  const int kind = (gather ? 2 : spill ? 1 : 0) + (paged ? 3 : 0);
  const int dt = dtype == KASCADE_F16 ? 2 : dtype == KASCADE_BF16 ? 1 : 0;
  int bpc;
  size_t st;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    int& b = d->splitk_bpc[dt][lg][kind];
    if (b == 0) {
      int n = 0;
      size_t sl = 0;
      hipError_t e = decode_splitk_attrs(dtype, G, gather, spill, paged, &n, &sl);
      if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return KASCADE_ERR_HIP;
      }
      b = n < 1 ? 1 : n;
      d->splitk_lds[dt][lg][kind] = sl;
    }
    bpc = b;
    st = d->splitk_lds[dt][lg][kind];
  }
  const size_t per_wg = st + decode_splitk_dyn_lds(dtype, G, gather, spill, paged, kps);
  if (per_wg > 0 && d->lds_per_cu > 0) {
    const int by_lds = (int)(d->lds_per_cu / per_wg);
    bpc = by_lds < bpc ? by_lds : bpc;
  }
  *slots = d->cus * (bpc < 1 ? 1 : bpc);
  return KASCADE_OK;
}

// ---- per-kernel event timing ------------------------------------------------
// Events are recorded around the launches of an enabled kernel; they are only
// waited for in kascade_kernel_timer_read, never in a launch call: when the
// pool is used up it grows (event creation is a host call and does not wait
// for the device).  A launch on a stream that is being captured into a graph
// is not timed (the events would become graph nodes).
struct Timer {
  std::atomic<bool> on{false};   // read by every launch, from any thread
  double total_ms = 0.0;
  int64_t launches = 0;
  std::vector<hipEvent_t> pool;   // pairs
  size_t used = 0;                // pairs recorded since the last drain
};
Timer g_timer[KASCADE_K_COUNT];
constexpr size_t kTimerPairs = 256;

hipError_t timer_grow(Timer& t) {
  const size_t old = t.pool.size();
  t.pool.resize(old + 2 * kTimerPairs, nullptr);
  for (size_t i = old; i < t.pool.size(); ++i) {
    hipError_t e = hipEventCreate(&t.pool[i]);
    if (e != hipSuccess) {
      for (size_t j = old; j < i; ++j) (void)hipEventDestroy(t.pool[j]);
      t.pool.resize(old);
      return e;
    }
  }
  return hipSuccess;
}

hipError_t timer_drain(Timer& t) {
  for (size_t i = 0; i < t.used; ++i) {
    hipError_t e = hipEventSynchronize(t.pool[2 * i + 1]);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.pool[2 * i], t.pool[2 * i + 1]);
    if (e != hipSuccess) return e;
    t.total_ms += ms;
    t.launches += 1;
  }
  t.used = 0;
  return hipSuccess;
}

template <typename F>
hipError_t timed(int id, hipStream_t s, F&& launch) {
  Timer& t = g_timer[id];
  if (!t.on.load(std::memory_order_relaxed)) return launch();
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return launch();
  if (2 * (t.used + 1) > t.pool.size()) {
    hipError_t e = timer_grow(t);
    if (e != hipSuccess) return e;
  }
  hipEvent_t b = t.pool[2 * t.used], en = t.pool[2 * t.used + 1];
  hipError_t e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(en, s);
  if (e != hipSuccess) return e;
  t.used += 1;
  return hipSuccess;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KASCADE_OK;
  g_last_hip_error = (int)e;
  return KASCADE_ERR_HIP;
}

// ---- validation ---------------------------------------------------------------
size_t elem_size(int dtype) { return dtype == KASCADE_F32 ? 4 : 2; }

// 64 rows of this many bytes span less than 2^31 bytes
constexpr int64_t kMaxPrefillRowBytes = ((int64_t)1 << 31) / 64;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const kascade_shape* s, bool prefill, bool paged = false) {
  if (!s) return KASCADE_ERR_NULL;
  if (s->reserved != 0) return KASCADE_ERR_ARG;
  if (s->batch < 1 || s->batch > 65535 || s->n_q_heads < 1 || s->n_kv_heads < 1 ||
      s->ctx_len < 1)
    return KASCADE_ERR_SHAPE;
  if (s->n_kv_heads > kMaxKvHeads || s->n_q_heads % s->n_kv_heads != 0) return KASCADE_ERR_SHAPE;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KASCADE_ERR_SHAPE;
  if (s->dtype == KASCADE_F32) {
    if (s->head_dim != 64 || prefill) return KASCADE_ERR_DTYPE;
  } else if (s->dtype == KASCADE_BF16 || s->dtype == KASCADE_F16) {
    if (s->head_dim != 128) return KASCADE_ERR_DTYPE;
  } else {
    return KASCADE_ERR_DTYPE;
  }
  if (!(s->scale >= 0.f) || isinf(s->scale)) return KASCADE_ERR_ARG;
  const int64_t es = (int64_t)elem_size(s->dtype);
  const int64_t d = s->head_dim;
  // every row must be 16-byte aligned and hold d elements; K/V rows are only
  // read, so any head/position interleaving works ([B,Hkv,N,d], [B,N,Hkv,d])
  if (s->kv_stride_n < d || s->q_stride_h < (prefill ? 0 : d)) return KASCADE_ERR_SHAPE;
  if ((s->kv_stride_n * es) % 16 || (s->kv_stride_h * es) % 16 || (s->kv_stride_b * es) % 16 ||
      (s->q_stride_h * es) % 16 || (s->q_stride_b * es) % 16 || (s->q_stride_n * es) % 16)
    return KASCADE_ERR_SHAPE;
  if (s->kv_stride_h < 0 || s->kv_stride_b < 0 || s->q_stride_b < 0 || s->q_stride_n < 0)
    return KASCADE_ERR_SHAPE;
  if (prefill && s->q_stride_n < d) return KASCADE_ERR_SHAPE;
  // decode kernels address a head's rows with 32-bit byte offsets
  if (!prefill && !paged && (int64_t)s->ctx_len * s->kv_stride_n * es > (int64_t)0xFFFFFF00)
    return KASCADE_ERR_SHAPE;
  // prefill kernels address the rows of a 64-key block with 32-bit byte
  // offsets from the block's first row
  if (prefill && s->kv_stride_n * es > kMaxPrefillRowBytes) return KASCADE_ERR_SHAPE;
  return KASCADE_OK;
}

float scale_log2(const kascade_shape* s) {
  const float sc = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  return sc * 1.4426950408889634f;
}

int check_rule(const kascade_topk_rule* r) {
  if (!r) return KASCADE_ERR_NULL;
  if (r->tile != 128 || r->pct < 1 || r->pct > 100 || r->round_to < 1 || r->k_min < 1)
    return KASCADE_ERR_TOPK;
  // every causal row must see at least one selected key (k_min >= tile)
  if (r->k_min < r->tile) return KASCADE_ERR_TOPK;
  return KASCADE_OK;
}

int check_head_map(const int32_t* hm, int n_kv, HeadMap* out) {
  if (!hm) return KASCADE_ERR_NULL;
  memset(out, 0, sizeof(*out));
  for (int g = 0; g < n_kv; ++g) {
    if (hm[g] < 0 || hm[g] >= n_kv) return KASCADE_ERR_HEADMAP;
    out->m[g] = hm[g];
  }
  return KASCADE_OK;
}

// ---- decode workspace -----------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecodePlan {
  int kps, splits;
  int wide_chunks;   // > 0: the anchor's select runs over chunks of many workgroups
  size_t off_hist, off_scores, off_part, off_lse2, off_pooled, total;
  size_t off_hist1, off_cand, off_chunk;
};

// Rows this long or longer are selected by the many-workgroup path.
constexpr int kWideMinKeys = 4096;
constexpr int kWideMaxChunks = 1024;

constexpr int kMinKeysPerSplit = 64;
constexpr int kMaxSplitsPerRow = 2048;   // the combine keeps one weight per split in LDS
constexpr int kMaxSlots = 2048;          // planning bound on resident workgroups

// Splits per (batch, KV head) row.  The grid is sized to whole rounds of the
// GPU's resident workgroup slots (a partial last round leaves most CUs idle
// while a few finish), with at most max_kps keys per split when that takes
// more than one round.  slots = 0 gives the largest split count any
// slots <= kMaxSlots can produce (workspace sizing).
int decode_splits(int64_t n_keys, int64_t rows, int slots, int64_t max_kps, int* kps_out) {
  int64_t S;
  if (slots <= 0) {
    S = kMaxSlots / rows + (n_keys + max_kps - 1) / max_kps;
  } else {
    const int64_t sl = slots > kMaxSlots ? kMaxSlots : slots;
    const int64_t total = n_keys * rows;
    const int64_t rounds = (total + sl * max_kps - 1) / (sl * max_kps);
    S = sl * rounds / rows;
  }
  S = S < 1 ? 1 : S;
  const int64_t min_kps = (n_keys + kMaxSplitsPerRow - 1) / kMaxSplitsPerRow;
  int64_t kps = (n_keys + S - 1) / S;
  kps = kps < min_kps ? min_kps : kps;
  kps = (kps + 15) / 16 * 16;              // whole load instructions for the 4 waves
  kps = kps < kMinKeysPerSplit ? kMinKeysPerSplit : kps;
  *kps_out = (int)kps;
  return (int)((n_keys + kps - 1) / kps);
}

// Passes without a score spill (reuse gather, dense): about two workgroups
// per CU, i.e. fewer and longer splits than the resident slots allow, which
// measured 3-6% faster (dense 128K: 16 splits of 8192 keys per row; the
// split merge reads fewer partials); a small gather keeps at least 64 keys
// per workgroup (one load step per wave: at 32K x 1, k 3264, 408 workgroups
// measured 10.1 us per reuse layer against 11.1 with 128 keys and 184
// workgroups; 48 or 32 keys were slower again).  Splits are capped at
// max_kps keys.
int decode_splits_target(int64_t n_keys, int64_t rows, int64_t target, int64_t max_kps,
                         int* kps_out) {
  int64_t S = target / rows;
  S = S < 1 ? 1 : S;
  int64_t kps = (n_keys + S - 1) / S;
  const int64_t min_kps = (n_keys + kMaxSplitsPerRow - 1) / kMaxSplitsPerRow;
  kps = kps < min_kps ? min_kps : kps;
  kps = (kps + 15) / 16 * 16;
  kps = kps < kMinKeysPerSplit ? kMinKeysPerSplit : kps;
  kps = kps > max_kps ? max_kps : kps;
  *kps_out = (int)kps;
  return (int)((n_keys + kps - 1) / kps);
}

int64_t decode_max_kps(const kascade_shape* s, bool spill, bool paged) {
  return spill && s->dtype != KASCADE_F32 ? spill_max_keys(s->n_q_heads / s->n_kv_heads, paged)
                                          : kPlanMaxKeys;
}

// target > 0: the split count of decode_splits_target for that many
// workgroups (max_kps_target keys at most), else the slot-based rule.
DecodePlan plan_decode(const kascade_shape* s, int n_keys, bool spill, bool pooled_ws,
                       int slots, int64_t target = 0, int64_t max_kps_target = 0, bool paged = false) {
  DecodePlan p;
  const int64_t rows = (int64_t)s->batch * s->n_kv_heads;
  const int64_t max_kps = decode_max_kps(s, spill, paged);
  p.splits = target > 0 ? decode_splits_target(n_keys, rows, target, max_kps_target, &p.kps)
                        : decode_splits(n_keys, rows, slots, max_kps, &p.kps);
  // the workspace always has room for the largest plan: the most splits come
  // with the smaller (paged) split cap, so a workspace sized here serves both
  int kps_max = 0;
  const int splits_ws = decode_splits(n_keys, rows, 0, decode_max_kps(s, spill, true), &kps_max);
  const int splits_room = splits_ws > p.splits ? splits_ws : p.splits;
  const int64_t BH = (int64_t)s->batch * s->n_q_heads;
  size_t off = 0;
  p.off_hist = off;
  if (spill) off += align256((size_t)rows * 2048 * 4);
  p.off_scores = off;
  if (spill) off += align256((size_t)BH * s->ctx_len * 4);
  p.off_part = off;
  off += align256((size_t)BH * splits_room * (s->head_dim + 2) * 4);
  p.off_lse2 = off;
  off += align256((size_t)BH * 4);
  p.off_pooled = off;
  if (pooled_ws) off += align256((size_t)rows * s->ctx_len * 4);
  p.wide_chunks = 0;
  p.off_hist1 = p.off_cand = p.off_chunk = 0;
  const int chunks = (s->ctx_len + wide_chunk(s->ctx_len) - 1) / wide_chunk(s->ctx_len);
  if (spill && s->ctx_len >= kWideMinKeys && chunks <= kWideMaxChunks) {
    p.wide_chunks = chunks;
    p.off_hist1 = off;
    off += align256((size_t)rows * 2048 * 4);
    p.off_cand = off;
    off += align256((size_t)rows * s->ctx_len * 4);
    p.off_chunk = off;
    off += align256((size_t)rows * chunks * 2 * 4);
  }
  p.total = off;
  return p;
}

// Plan with the slots the variant leaves at the largest split, then once more
// if the planned split needs less LDS and so leaves more slots.
int plan_decode_dev(DeviceInfo* d, const kascade_shape* s, int n_keys, bool gather, bool spill,
                    bool pooled_ws, bool paged, DecodePlan* p) {
  const int G = s->n_q_heads / s->n_kv_heads;
  if (!spill) {
    const int64_t total = (int64_t)n_keys * s->batch * s->n_kv_heads;
    int64_t target = 2 * (int64_t)(d->cus > 0 ? d->cus : 1);
    if (gather) target = total / 64 < target ? (total / 64 > 0 ? total / 64 : 1) : target;
    *p = plan_decode(s, n_keys, spill, pooled_ws, 0, target,
                     (gather || paged) ? kMaxGatherKeys : (int64_t)1 << 30);
    return KASCADE_OK;
  }
  int slots = 0, st;
  if ((st = splitk_slots(d, s->dtype, G, gather, spill, paged, (int)decode_max_kps(s, spill, paged),
                         &slots)))
    return st;
  *p = plan_decode(s, n_keys, spill, pooled_ws, slots, 0, 0, paged);
  int slots2 = 0;
  if ((st = splitk_slots(d, s->dtype, G, gather, spill, paged, p->kps, &slots2))) return st;
  if (slots2 > slots) *p = plan_decode(s, n_keys, spill, pooled_ws, slots2, 0, 0, paged);
  return KASCADE_OK;
}

DecodeArgs decode_args(const kascade_shape* s, const void* q, const void* k, const void* v,
                       int n_keys, const DecodePlan& p, char* ws) {
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_sb = s->q_stride_b;
  a.q_sh = s->q_stride_h;
  a.kv_sb = s->kv_stride_b;
  a.kv_sh = s->kv_stride_h;
  a.kv_sn = s->kv_stride_n;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.n_keys = n_keys;
  a.n_ctx = s->ctx_len;
  a.scale_log2 = scale_log2(s);
  a.keys_per_split = p.kps;
  a.n_splits = p.splits;
  a.part = reinterpret_cast<float*>(ws + p.off_part);
  return a;
}

// ---- prefill workspace -----------------------------------------------------------
int64_t packed_per_batch(const kascade_shape* s, int tile) {
  const int T = (s->ctx_len + tile - 1) / tile;
  return packed_row_offset(T, 0, s->n_kv_heads, tile, s->ctx_len);
}

struct PrefillPlan {
  size_t off_lse2, off_pooled, total;
};

PrefillPlan plan_prefill(const kascade_shape* s, const kascade_topk_rule* r, bool pooled_ws) {
  PrefillPlan p;
  size_t off = 0;
  p.off_lse2 = off;
  off += align256((size_t)s->batch * s->n_q_heads * s->ctx_len * 4);
  p.off_pooled = off;
  if (pooled_ws) off += align256((size_t)s->batch * packed_per_batch(s, r->tile) * 4);
  p.total = off;
  return p;
}

PrefillArgs prefill_args(const kascade_shape* s, const void* q, const void* k, const void* v,
                         void* out) {
  PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_sb = s->q_stride_b;
  a.q_sh = s->q_stride_h;
  a.q_sn = s->q_stride_n;
  a.kv_sb = s->kv_stride_b;
  a.kv_sh = s->kv_stride_h;
  a.kv_sn = s->kv_stride_n;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.N = s->ctx_len;
  a.T = (s->ctx_len + 127) / 128;
  a.scale_log2 = scale_log2(s);
  a.half = s->dtype == KASCADE_F16 ? 1 : 0;
  a.out = out;
  return a;
}

}  // namespace

// ---- fused anchor decode workspace ----------------------------------------------
// [status word, 256 B][row barrier counters of kFusedMaxRows rows][partials
// for up to kFusedMaxSplits splits][hist0][hist1][candidates][split counts].
// The state (status word and counters) sits at the same offsets for every
// shape, so a workspace serves calls of different shapes; it must be zero
// before the first call and every call leaves the counters zero (a call that
// gave up waiting sets status bit 0).
constexpr int kFusedMaxSplits = 256;            // one split per thread of the select phases
constexpr int kFusedMaxRows = 256;              // rows x splits <= resident workgroups
constexpr uint32_t kFusedDefaultPolls = 1u << 18;

struct FusedPlan {
  size_t off_status, off_sync, off_part, off_hist0, off_hist1, off_cand, off_cnt, total;
};

FusedPlan plan_fused(const kascade_shape* s) {
  FusedPlan p;
  const size_t rows = (size_t)s->batch * s->n_kv_heads, BH = (size_t)s->batch * s->n_q_heads;
  size_t o = 0;
  p.off_status = o;
  o += 256;
  p.off_sync = o;
  o += align256((size_t)kFusedMaxRows * kFusedSyncWords * 4);
  p.off_part = o;
  o += align256(BH * kFusedMaxSplits * (size_t)(s->head_dim + 2) * 4);
  p.off_hist0 = o;
  o += align256(rows * 2048 * 4);
  p.off_hist1 = o;
  o += align256(rows * 2048 * 4);
  p.off_cand = o;
  o += align256(rows * (size_t)s->ctx_len * 4);
  p.off_cnt = o;
  o += align256(rows * kFusedMaxSplits * 2 * 4);
  p.total = o;
  return p;
}

extern "C" {

const char* kascade_version(void) { return "kascade-mi355x 0.1"; }

int kascade_last_hip_error(void) { return g_last_hip_error; }

const char* kascade_status_str(int st) {
  switch (st) {
    case KASCADE_OK: return "ok";
    case KASCADE_ERR_NULL: return "null pointer";
    case KASCADE_ERR_SHAPE: return "unsupported or inconsistent shape/strides";
    case KASCADE_ERR_DTYPE: return "unsupported dtype/head_dim";
    case KASCADE_ERR_TOPK: return "topk out of range or invalid rule";
    case KASCADE_ERR_HEADMAP: return "head_map entry out of range";
    case KASCADE_ERR_WORKSPACE: return "workspace too small";
    case KASCADE_ERR_HIP: return "HIP error";
    case KASCADE_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

int32_t kascade_topk_for_len(int32_t n, const kascade_topk_rule* rule) {
  if (!rule || rule->pct < 1 || rule->pct > 100 || rule->round_to < 1 || rule->k_min < 1 || n < 0)
    return -1;
  return tile_k_for_len(n, rule->pct, rule->round_to, rule->k_min);
}

size_t kascade_workspace_bytes(int op, const kascade_shape* s, int32_t topk,
                               const kascade_topk_rule* rule) {
  const bool prefill = op == 2 || op == 3 || op == 5;
  // sizes depend on the dimensions only (decode: paged caches too)
  if (check_shape(s, prefill, !prefill) != KASCADE_OK) return 0;
  switch (op) {
    case 0: return plan_decode(s, s->ctx_len, true, true, 0).total;
    case 1: return topk >= 1 ? plan_decode(s, topk, false, false, 0).total : 0;
    case 4: return plan_decode(s, s->ctx_len, false, false, 0).total;
    case 6: return plan_fused(s).total;
    case 2: return check_rule(rule) == KASCADE_OK ? plan_prefill(s, rule, true).total : 0;
    case 3: return 0;
    case 5: return 0;
  }
  return 0;
}

// A paged cache descriptor, checked against the shape.
static int check_paged(const kascade_shape* s, const kascade_paged_kv* pg) {
  if (!pg) return KASCADE_OK;
  if (!pg->block_table) return KASCADE_ERR_NULL;
  if (pg->reserved != 0) return KASCADE_ERR_ARG;
  if (s->dtype == KASCADE_F32) return KASCADE_ERR_DTYPE;
  const int bs = pg->block_size;
  if (bs < 1 || bs > (1 << 20) || (bs & (bs - 1)) != 0 || pg->num_blocks < 1) return KASCADE_ERR_SHAPE;
  if ((int64_t)pg->table_stride < ((int64_t)s->ctx_len + bs - 1) / bs) return KASCADE_ERR_SHAPE;
  if (pg->block_stride <= 0 || pg->block_stride % s->kv_stride_n != 0 ||
      (pg->block_stride * 2) % 16 != 0)
    return KASCADE_ERR_SHAPE;
  // every head's rows stay inside the block; physical row numbers fit 32 bits
  if ((int64_t)(s->n_kv_heads - 1) * s->kv_stride_h + (int64_t)(bs - 1) * s->kv_stride_n +
          s->head_dim > pg->block_stride)
    return KASCADE_ERR_SHAPE;
  if ((int64_t)pg->num_blocks * (pg->block_stride / s->kv_stride_n) > (int64_t)0xFFFFFFF0)
    return KASCADE_ERR_SHAPE;
  return KASCADE_OK;
}

static void set_paged(DecodeArgs& a, const kascade_shape* s, const kascade_paged_kv* pg) {
  if (!pg) return;
  a.table = pg->block_table;
  a.table_stride = pg->table_stride;
  int sh = 0;
  while ((1 << sh) < pg->block_size) ++sh;
  a.blk_shift = sh;
  a.num_blocks = pg->num_blocks;
  a.blk_rows = pg->block_stride / s->kv_stride_n;
}

static int anchor_decode_impl(const kascade_shape* s, const kascade_paged_kv* pg, const void* q,
                       const void* k, const void* v, int32_t topk, void* out, float* lse_out,
                       int32_t* topk_idx, float* pooled_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  int st = check_shape(s, false, pg != nullptr);
  if (st) return st;
  if ((st = check_paged(s, pg))) return st;
  if (!q || !k || !v || !out || !topk_idx) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return KASCADE_ERR_ARG;
  if (topk < 1 || topk > s->ctx_len) return KASCADE_ERR_TOPK;
  if (!ws || ws_bytes < plan_decode(s, s->ctx_len, true, true, 0).total)
    return KASCADE_ERR_WORKSPACE;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  DecodePlan p;
  if ((st = plan_decode_dev(dev, s, s->ctx_len, false, true, true, pg != nullptr, &p))) return st;
  if (p.kps > decode_max_kps(s, true, pg != nullptr)) return KASCADE_ERR_SHAPE;   // LDS score buffer
  char* w = reinterpret_cast<char*>(ws);
  DecodeArgs a = decode_args(s, q, k, v, s->ctx_len, p, w);
  set_paged(a, s, pg);
  a.scores = reinterpret_cast<float*>(w + p.off_scores);
  a.hist0 = reinterpret_cast<uint32_t*>(w + p.off_hist);
  if (p.wide_chunks) {
    a.hist1 = reinterpret_cast<uint32_t*>(w + p.off_hist1);
  }
  float* pooled = pooled_out ? pooled_out : reinterpret_cast<float*>(w + p.off_pooled);
  hipError_t e = timed(KASCADE_K_DECODE_SPLITK, stream,
                       [&] { return launch_decode_splitk(a, s->dtype, false, stream); });
  if (e != hipSuccess) return hip_status(e);
  // one launch pools the row (its lse from the splits' (m, l)) and merges the
  // splits into out / lse_out
  PoolDecodeArgs pa;
  memset(&pa, 0, sizeof(pa));
  pa.scores = a.scores;
  pa.part = a.part;
  pa.n_splits = p.splits;
  pa.pooled = pooled;
  pa.hist0 = a.hist0;
  pa.out = out;
  pa.lse_out = lse_out;
  pa.B = s->batch;
  pa.Hq = s->n_q_heads;
  pa.Hkv = s->n_kv_heads;
  pa.N = s->ctx_len;
  e = timed(KASCADE_K_DECODE_POOL, stream, [&] { return launch_decode_pool(pa, s->dtype, stream); });
  if (e != hipSuccess) return hip_status(e);
  if (p.wide_chunks) {
    WideSelectArgs wa;
    memset(&wa, 0, sizeof(wa));
    wa.src = pooled;
    wa.row_stride = s->ctx_len;
    wa.rows = s->batch * s->n_kv_heads;
    wa.n = s->ctx_len;
    wa.k = topk;
    wa.chunks = p.wide_chunks;
    wa.idx = topk_idx;
    wa.idx_stride = topk;
    wa.hist0 = a.hist0;
    wa.hist1 = a.hist1;
    wa.cand = reinterpret_cast<uint32_t*>(w + p.off_cand);
    wa.chunk_cnt = reinterpret_cast<uint32_t*>(w + p.off_chunk);
    e = timed(KASCADE_K_TOPK_SELECT, stream, [&] { return launch_topk_select_wide(wa, stream); });
    return hip_status(e);
  }
  SelectArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.src = pooled;
  sa.row_stride = s->ctx_len;
  sa.rows = s->batch * s->n_kv_heads;
  sa.n = s->ctx_len;
  sa.k = topk;
  sa.idx = topk_idx;
  sa.idx_stride = topk;
  sa.mode = 0;
  sa.cache_cap = dev->select_cache_cap;
  sa.hist0 = a.hist0;
  e = timed(KASCADE_K_TOPK_SELECT, stream, [&] { return launch_topk_select(sa, stream); });
  return hip_status(e);
}

// use_scratch: the partials and lse go to this GPU's scratch array (laid out
// for the planned split count) instead of the caller's workspace.
static int reuse_decode_impl(const kascade_shape* s, const kascade_paged_kv* pg, const void* q,
                      const void* k, const void* v, int32_t topk, const int32_t* idx,
                      const int32_t* head_map, void* out, void* ws, size_t ws_bytes,
                      hipStream_t stream, bool use_scratch = false) {
  int st = check_shape(s, false, pg != nullptr);
  if (st) return st;
  if ((st = check_paged(s, pg))) return st;
  if (!q || !k || !v || !out || !idx) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return KASCADE_ERR_ARG;
  if (topk < 1 || topk > s->ctx_len) return KASCADE_ERR_TOPK;
  HeadMap hm;
  if ((st = check_head_map(head_map, s->n_kv_heads, &hm))) return st;
  if (!use_scratch && (!ws || ws_bytes < plan_decode(s, topk, false, false, 0).total))
    return KASCADE_ERR_WORKSPACE;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  DecodePlan p;
  if ((st = plan_decode_dev(dev, s, topk, true, false, false, pg != nullptr, &p))) return st;
  if (p.kps > kMaxGatherKeys) return KASCADE_ERR_SHAPE;
  if (use_scratch) {
    // partials [B*Hq, splits, d+2] then log2-lse [B*Hq], all fp32
    const size_t BH = (size_t)s->batch * s->n_q_heads;
    p.off_part = 0;
    p.off_lse2 = align256(BH * (size_t)p.splits * (size_t)(s->head_dim + 2) * 4);
    p.total = p.off_lse2 + align256(BH * 4);
    if (p.total > kScratchBytes) return KASCADE_ERR_WORKSPACE;
    ws = dev->scratch;
  }
  char* w = reinterpret_cast<char*>(ws);
  DecodeArgs a = decode_args(s, q, k, v, topk, p, w);
  set_paged(a, s, pg);
  a.idx = idx;
  a.idx_sg = topk;
  a.idx_sb = (int64_t)s->n_kv_heads * topk;
  a.hm = hm;
  hipError_t e = timed(KASCADE_K_REUSE_DECODE, stream,
                       [&] { return launch_decode_splitk(a, s->dtype, true, stream); });
  if (e != hipSuccess) return hip_status(e);
  CombineArgs c = {a.part, p.splits, s->batch * s->n_q_heads, out,
                   reinterpret_cast<float*>(w + p.off_lse2), nullptr};
  e = timed(KASCADE_K_DECODE_COMBINE, stream,
            [&] { return launch_decode_combine(c, s->dtype, stream); });
  return hip_status(e);
}

int kascade_anchor_decode(const kascade_shape* s, const void* q, const void* k, const void* v,
                          int32_t topk, void* out, float* lse_out, int32_t* topk_idx,
                          float* pooled_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return anchor_decode_impl(s, nullptr, q, k, v, topk, out, lse_out, topk_idx, pooled_out, ws,
                            ws_bytes, stream);
}

int kascade_anchor_decode_fused(const kascade_shape* s, const void* q, const void* k,
                                const void* v, int32_t topk, void* out, float* lse_out,
                                int32_t* topk_idx, float* pooled_out, uint32_t max_polls, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(s, false);
  if (st) return st;
  if (s->dtype == KASCADE_F32) return KASCADE_ERR_DTYPE;
  if (!q || !k || !v || !out || !topk_idx) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return KASCADE_ERR_ARG;
  if (topk < 1 || topk > s->ctx_len) return KASCADE_ERR_TOPK;
  const FusedPlan fp = plan_fused(s);
  if (!ws || ws_bytes < fp.total) return KASCADE_ERR_WORKSPACE;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  // the split plan of the spilling anchor pass (so the two paths split alike)
  DecodePlan p;
  if ((st = plan_decode_dev(dev, s, s->ctx_len, false, true, true, false, &p))) return st;
  if (p.kps > decode_max_kps(s, true, false) || p.splits > kFusedMaxSplits) return KASCADE_ERR_SHAPE;
  // every workgroup must be resident at once: the row barriers wait for all
  // of a row's splits
  const int G = s->n_q_heads / s->n_kv_heads;
  int blocks = 0;
  size_t static_lds = 0;
  hipError_t e = anchor_fused_attrs(s->dtype, G, p.kps, &blocks, &static_lds);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return KASCADE_ERR_HIP;
  }
  const int64_t rows = (int64_t)s->batch * s->n_kv_heads;
  if (rows > kFusedMaxRows || rows * p.splits > (int64_t)dev->cus * blocks) return KASCADE_ERR_SHAPE;
  if (dev->lds_per_cu > 0 && static_lds + anchor_fused_dyn_lds(G, p.kps) > dev->lds_per_cu)
    return KASCADE_ERR_SHAPE;
  char* w = reinterpret_cast<char*>(ws);
  FusedDecodeArgs f;
  memset(&f, 0, sizeof(f));
  f.d = decode_args(s, q, k, v, s->ctx_len, p, w);
  f.d.part = reinterpret_cast<float*>(w + fp.off_part);
  f.out = out;
  f.lse_out = lse_out;
  f.idx = topk_idx;
  f.pooled = pooled_out;
  f.k = topk;
  f.sync = reinterpret_cast<uint32_t*>(w + fp.off_sync);
  f.status = reinterpret_cast<uint32_t*>(w + fp.off_status);
  f.spin_limit = max_polls ? max_polls : kFusedDefaultPolls;
  f.hist0 = reinterpret_cast<uint32_t*>(w + fp.off_hist0);
  f.hist1 = reinterpret_cast<uint32_t*>(w + fp.off_hist1);
  f.cand = reinterpret_cast<uint32_t*>(w + fp.off_cand);
  f.cnt = reinterpret_cast<uint32_t*>(w + fp.off_cnt);
  f.cand_cap = (uint32_t)(anchor_fused_dyn_lds(G, p.kps) / sizeof(uint32_t)) - (uint32_t)p.kps;
  e = timed(KASCADE_K_ANCHOR_FUSED, stream, [&] { return launch_anchor_fused(f, s->dtype, stream); });
  return hip_status(e);
}

int kascade_reuse_decode(const kascade_shape* s, const void* q, const void* k, const void* v,
                         int32_t topk, const int32_t* idx, const int32_t* head_map, void* out,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  return reuse_decode_impl(s, nullptr, q, k, v, topk, idx, head_map, out, ws, ws_bytes, stream);
}

int kascade_reuse_decode_noalloc(const kascade_shape* s, const void* q, const void* k,
                                 const void* v, int32_t topk, const int32_t* idx,
                                 const int32_t* head_map, void* out, hipStream_t stream) {
  return reuse_decode_impl(s, nullptr, q, k, v, topk, idx, head_map, out, nullptr, 0, stream, true);
}

int kascade_anchor_decode_paged(const kascade_shape* s, const kascade_paged_kv* paged,
                                const void* q, const void* k_cache, const void* v_cache,
                                int32_t topk, void* out, float* lse_out, int32_t* topk_idx,
                                float* pooled_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!paged) return KASCADE_ERR_NULL;
  return anchor_decode_impl(s, paged, q, k_cache, v_cache, topk, out, lse_out, topk_idx,
                            pooled_out, ws, ws_bytes, stream);
}

int kascade_reuse_decode_paged(const kascade_shape* s, const kascade_paged_kv* paged,
                               const void* q, const void* k_cache, const void* v_cache,
                               int32_t topk, const int32_t* anchor_topk_idx,
                               const int32_t* head_map, void* out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!paged) return KASCADE_ERR_NULL;
  return reuse_decode_impl(s, paged, q, k_cache, v_cache, topk, anchor_topk_idx, head_map, out, ws,
                           ws_bytes, stream);
}

int kascade_dense_decode(const kascade_shape* s, const void* q, const void* k, const void* v,
                         void* out, float* lse_out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  int st = check_shape(s, false);
  if (st) return st;
  if (!q || !k || !v || !out) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return KASCADE_ERR_ARG;
  if (!ws || ws_bytes < plan_decode(s, s->ctx_len, false, false, 0).total)
    return KASCADE_ERR_WORKSPACE;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  DecodePlan p;
  if ((st = plan_decode_dev(dev, s, s->ctx_len, false, false, false, false, &p))) return st;
  char* w = reinterpret_cast<char*>(ws);
  DecodeArgs a = decode_args(s, q, k, v, s->ctx_len, p, w);
  hipError_t e = timed(KASCADE_K_DECODE_SPLITK, stream,
                       [&] { return launch_decode_splitk(a, s->dtype, false, stream); });
  if (e != hipSuccess) return hip_status(e);
  CombineArgs c = {a.part, p.splits, s->batch * s->n_q_heads, out,
                   reinterpret_cast<float*>(w + p.off_lse2), lse_out};
  e = timed(KASCADE_K_DECODE_COMBINE, stream,
            [&] { return launch_decode_combine(c, s->dtype, stream); });
  return hip_status(e);
}

// ---- calibration -------------------------------------------------------------

int kascade_calib_head_similarity(int32_t L, int32_t S, int32_t n_kv_heads, int32_t n, int32_t k,
                                  const float* pooled, const int32_t* topk_idx, float* sim,
                                  hipStream_t stream) {
  if (!pooled || !topk_idx || !sim) return KASCADE_ERR_NULL;
  if (L < 1 || L > 65535 || S < 1 || n_kv_heads < 1 || n_kv_heads > kMaxKvHeads || n < 1)
    return KASCADE_ERR_SHAPE;
  if (k < 1 || k > n) return KASCADE_ERR_TOPK;
  return hip_status(launch_calib_sim(pooled, topk_idx, L, S, n_kv_heads, n, k, sim, stream));
}

size_t kascade_layer_weight_workspace_bytes(int32_t tokens) {
  return tokens < 1 ? 0 : (size_t)((tokens + 63) / 64) * sizeof(double);
}

int kascade_layer_weight(const void* x, const void* y, int32_t tokens, int32_t dim, int32_t dtype,
                         float* w_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !y || !w_out) return KASCADE_ERR_NULL;
  if (tokens < 1 || dim < 1) return KASCADE_ERR_SHAPE;
  if (dtype != KASCADE_F32 && dtype != KASCADE_BF16 && dtype != KASCADE_F16) return KASCADE_ERR_DTYPE;
  if (!workspace || workspace_bytes < kascade_layer_weight_workspace_bytes(tokens))
    return KASCADE_ERR_WORKSPACE;
  return hip_status(launch_layer_weight(x, y, tokens, dim, dtype, reinterpret_cast<double*>(workspace),
                                        w_out, stream));
}

int kascade_weighted_similarity(int32_t L, int32_t n_kv_heads, const float* sim, const float* w,
                                double* S) {
  if (!sim || !S) return KASCADE_ERR_NULL;
  if (L < 1 || n_kv_heads < 1) return KASCADE_ERR_SHAPE;
  const int H = n_kv_heads;
  for (int a = 0; a < L; ++a) {
    for (int b = 0; b < L; ++b) {
      if (b < a) {
        S[(int64_t)a * L + b] = 0.0;
        continue;
      }
      // mean over b's heads of their best (lowest ga on ties) anchor head
      double tot = 0.0;
      for (int gb = 0; gb < H; ++gb) {
        const float* col = sim + ((int64_t)a * L + b) * H * H + gb;
        float best = col[0];
        for (int ga = 1; ga < H; ++ga) best = col[(int64_t)ga * H] > best ? col[(int64_t)ga * H] : best;
        tot += (double)best;
      }
      S[(int64_t)a * L + b] = (w ? (double)w[b] : 1.0) * (tot / H);
    }
  }
  return KASCADE_OK;
}

int kascade_select_anchors(int32_t L, int32_t M, const double* S, int32_t* anchors, double* score) {
  if (!S || !anchors) return KASCADE_ERR_NULL;
  if (L < 1 || M < 1 || M > L) return KASCADE_ERR_ARG;
  // pref[i][j] = sum_{l=i}^{j-1} S[i][l]: the similarity layers i..j-1 keep when i anchors them
  std::vector<double> pref((size_t)L * (L + 1), 0.0);
  for (int i = 0; i < L; ++i) {
    double acc = 0.0;
    for (int j = i; j < L; ++j) {
      acc += S[(int64_t)i * L + j];
      pref[(size_t)i * (L + 1) + j + 1] = acc;
    }
  }
  const double NEG = -HUGE_VAL;
  std::vector<double> dp((size_t)(M + 1) * (L + 1), NEG);
  std::vector<int32_t> arg((size_t)(M + 1) * (L + 1), -1);
  dp[0] = 0.0;
  for (int m = 1; m <= M; ++m) {
    for (int j = m; j <= L; ++j) {
      double best = NEG;
      int bi = -1;
      for (int i = m - 1; i < j; ++i) {   // the last segment [i, j) starts at anchor i
        const double prev = dp[(size_t)(m - 1) * (L + 1) + i];
        if (prev == NEG) continue;
        const double v = prev + pref[(size_t)i * (L + 1) + j];
        if (v > best) {
          best = v;
          bi = i;
        }
      }
      dp[(size_t)m * (L + 1) + j] = best;
      arg[(size_t)m * (L + 1) + j] = bi;
    }
  }
  int j = L;
  for (int m = M; m >= 1; --m) {
    const int i = arg[(size_t)m * (L + 1) + j];
    anchors[m - 1] = i;
    j = i;
  }
  if (score) *score = dp[(size_t)M * (L + 1) + L];
  return KASCADE_OK;
}

int kascade_head_maps(int32_t L, int32_t n_kv_heads, const float* sim, const int32_t* anchors,
                      int32_t M, int32_t* head_maps) {
  if (!sim || !anchors || !head_maps) return KASCADE_ERR_NULL;
  if (L < 1 || n_kv_heads < 1 || M < 1 || M > L) return KASCADE_ERR_ARG;
  if (anchors[0] != 0) return KASCADE_ERR_ARG;
  for (int m = 1; m < M; ++m)
    if (anchors[m] <= anchors[m - 1] || anchors[m] >= L) return KASCADE_ERR_ARG;
  const int H = n_kv_heads;
  int a = 0, next = 1;
  for (int b = 0; b < L; ++b) {
    if (next < M && anchors[next] == b) {
      a = b;
      ++next;
    }
    for (int gb = 0; gb < H; ++gb) {
      if (b == a) {
        head_maps[(int64_t)b * H + gb] = gb;
        continue;
      }
      const float* col = sim + ((int64_t)a * L + b) * H * H + gb;
      int best = 0;
      for (int ga = 1; ga < H; ++ga)
        if (col[(int64_t)ga * H] > col[(int64_t)best * H]) best = ga;
      head_maps[(int64_t)b * H + gb] = best;
    }
  }
  return KASCADE_OK;
}

int kascade_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return KASCADE_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || !aligned16(src) || ((uintptr_t)sink & 3u) != 0) return KASCADE_ERR_ARG;
  DeviceInfo* dev = nullptr;
  int st = device_setup(&dev);
  if (st) return st;
  // one 1024-thread workgroup per CU, each streaming a contiguous range
  const int grid = dev->cus > 0 ? dev->cus : 1;
  return hip_status(launch_stream_read(src, (int64_t)(bytes / 16), sink, grid, stream));
}

int kascade_topk_select_f32(const float* scores, int64_t row_stride, int32_t rows, int32_t n,
                            int32_t k, int32_t* idx, int64_t idx_stride, hipStream_t stream) {
  if (!scores || !idx) return KASCADE_ERR_NULL;
  if (rows < 0 || rows > 2147483647 / 2 || n < 1 || row_stride < n) return KASCADE_ERR_SHAPE;
  if (k < 1 || k > n || idx_stride < k) return KASCADE_ERR_TOPK;
  if (rows == 0) return KASCADE_OK;
  DeviceInfo* dev = nullptr;
  int st = device_setup(&dev);
  if (st) return st;
  SelectArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.src = scores;
  sa.row_stride = row_stride;
  sa.rows = rows;
  sa.n = n;
  sa.k = k;
  sa.idx = idx;
  sa.idx_stride = idx_stride;
  sa.mode = 0;
  sa.cache_cap = dev->select_cache_cap;
  return hip_status(timed(KASCADE_K_TOPK_SELECT, stream,
                          [&] { return launch_topk_select(sa, stream); }));
}

int kascade_anchor_prefill(const kascade_shape* s, const void* q, const void* k, const void* v,
                           const kascade_topk_rule* rule, void* out, float* lse_out,
                           int32_t* tile_idx, float* pooled_out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int st = check_shape(s, true);
  if (st) return st;
  if ((st = check_rule(rule))) return st;
  if (!q || !k || !v || !out || !tile_idx) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KASCADE_ERR_ARG;
  const PrefillPlan p = plan_prefill(s, rule, pooled_out == nullptr);
  if (!ws || ws_bytes < p.total) return KASCADE_ERR_WORKSPACE;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  char* w = reinterpret_cast<char*>(ws);
  PrefillArgs a = prefill_args(s, q, k, v, out);
  a.lse2 = reinterpret_cast<float*>(w + p.off_lse2);
  a.lse_out = lse_out;
  a.pooled = pooled_out ? pooled_out : reinterpret_cast<float*>(w + p.off_pooled);
  a.packed_per_batch = packed_per_batch(s, rule->tile);
  hipError_t e = timed(KASCADE_K_PREFILL_FLASH, stream, [&] { return launch_prefill_flash(a, stream); });
  if (e != hipSuccess) return hip_status(e);
  e = timed(KASCADE_K_PREFILL_POOL, stream, [&] { return launch_prefill_pool(a, stream); });
  if (e != hipSuccess) return hip_status(e);
  SelectArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.src = a.pooled;
  sa.rows = s->batch * a.T * s->n_kv_heads;
  sa.idx = tile_idx;
  sa.idx_stride = tile_k_for_len(s->ctx_len, rule->pct, rule->round_to, rule->k_min);
  sa.mode = 1;
  sa.T = a.T;
  sa.Hkv = s->n_kv_heads;
  sa.N = s->ctx_len;
  sa.tile = rule->tile;
  sa.pct = rule->pct;
  sa.round_to = rule->round_to;
  sa.k_min = rule->k_min;
  sa.packed_per_batch = a.packed_per_batch;
  sa.cache_cap = dev->select_cache_cap;
  e = timed(KASCADE_K_TOPK_SELECT, stream, [&] { return launch_topk_select(sa, stream); });
  return hip_status(e);
}

static int reuse_prefill_impl(const kascade_shape* s, const kascade_paged_kv* pg, const void* q,
                              const void* k, const void* v, const kascade_topk_rule* rule,
                              const int32_t* idx, const int32_t* head_map, void* out,
                              hipStream_t stream) {
  int st = check_shape(s, true, pg != nullptr);
  if (st) return st;
  if ((st = check_paged(s, pg))) return st;
  if ((st = check_rule(rule))) return st;
  if (!q || !k || !v || !out || !idx) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KASCADE_ERR_ARG;
  HeadMap hm;
  if ((st = check_head_map(head_map, s->n_kv_heads, &hm))) return st;
  const size_t max_list = pg ? prefill_sparse_paged_max_list() : prefill_sparse_max_list();
  if ((size_t)tile_k_for_len(s->ctx_len, rule->pct, rule->round_to, rule->k_min) > max_list)
    return KASCADE_ERR_SHAPE;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  PrefillArgs a = prefill_args(s, q, k, v, out);
  a.idx = idx;
  a.k_max = tile_k_for_len(s->ctx_len, rule->pct, rule->round_to, rule->k_min);
  a.pct = rule->pct;
  a.round_to = rule->round_to;
  a.k_min = rule->k_min;
  a.hm = hm;
  if (pg) {
    a.table = pg->block_table;
    a.table_stride = pg->table_stride;
    int sh = 0;
    while ((1 << sh) < pg->block_size) ++sh;
    a.blk_shift = sh;
    a.num_blocks = pg->num_blocks;
    a.blk_rows = (uint32_t)(pg->block_stride / s->kv_stride_n);
  }
  return hip_status(timed(KASCADE_K_PREFILL_SPARSE, stream,
                          [&] { return launch_prefill_sparse(a, stream); }));
}

int kascade_reuse_prefill(const kascade_shape* s, const void* q, const void* k, const void* v,
                          const kascade_topk_rule* rule, const int32_t* idx,
                          const int32_t* head_map, void* out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return reuse_prefill_impl(s, nullptr, q, k, v, rule, idx, head_map, out, stream);
}

int kascade_reuse_prefill_paged(const kascade_shape* s, const kascade_paged_kv* pg, const void* q,
                                const void* k_cache, const void* v_cache,
                                const kascade_topk_rule* rule, const int32_t* idx,
                                const int32_t* head_map, void* out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!pg) return KASCADE_ERR_NULL;
  return reuse_prefill_impl(s, pg, q, k_cache, v_cache, rule, idx, head_map, out, stream);
}

int kascade_dense_prefill(const kascade_shape* s, const void* q, const void* k, const void* v,
                          void* out, float* lse_out, hipStream_t stream) {
  int st = check_shape(s, true);
  if (st) return st;
  if (!q || !k || !v || !out) return KASCADE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return KASCADE_ERR_ARG;
  DeviceInfo* dev = nullptr;
  if ((st = device_setup(&dev))) return st;
  PrefillArgs a = prefill_args(s, q, k, v, out);
  a.lse_out = lse_out;
  return hip_status(timed(KASCADE_K_PREFILL_FLASH, stream,
                          [&] { return launch_prefill_flash(a, stream); }));
}

int kascade_kernel_timer_enable(int id, int enable) {
  if (id < 0 || id >= KASCADE_K_COUNT) return KASCADE_ERR_ARG;
  Timer& t = g_timer[id];
  if (enable) {
    if (t.pool.empty()) {
      hipError_t e = timer_grow(t);
      if (e != hipSuccess) return hip_status(e);
    }
    t.used = 0;
    t.total_ms = 0.0;
    t.launches = 0;
  }
  t.on.store(enable != 0, std::memory_order_relaxed);
  return KASCADE_OK;
}

int kascade_kernel_timer_read(int id, double* total_ms, int64_t* launches) {
  if (id < 0 || id >= KASCADE_K_COUNT) return KASCADE_ERR_ARG;
  if (!total_ms || !launches) return KASCADE_ERR_NULL;
  Timer& t = g_timer[id];
  hipError_t e = timer_drain(t);
  if (e != hipSuccess) return hip_status(e);
  *total_ms = t.total_ms;
  *launches = t.launches;
  return KASCADE_OK;
}

}  // extern "C"
