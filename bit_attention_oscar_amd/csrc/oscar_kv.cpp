// Host side of the OSCAR INT2 KV library: argument validation, device memory,
// the split plan of decode attention and the kernel launches.  Every launch
// goes onto the caller's stream; nothing on the append/decode path
// synchronises the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/oscar_kv.h"
#include "common.h"
#include "prefill_attn.h"

using namespace oscar;

static_assert(sizeof(oscar_kv_dtype) == sizeof(int32_t), "enum fields of the config are 32-bit");

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t _e = (expr);                                                             \
    if (_e != hipSuccess)                                                               \
      return fail(OSCAR_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(_e));    \
  } while (0)

struct Plane {
  uint8_t* codes = nullptr;
  uint32_t* meta = nullptr;
  uint16_t* sink = nullptr;
  uint16_t* ring = nullptr;
  uint16_t* full = nullptr;
  float* smax = nullptr;
};

// Token counts of a layer: every sequence has its own (lens, host side; the
// host issues every append, so it knows them without reading the device).
// T is the longest.  dlens is the device copy the kernels of a ragged batch
// read; it matches lens for sequences [0, dev_synced).
struct Layer {
  Plane k, v;
  int32_t T = 0;
  std::vector<int32_t> lens;
  int* dlens = nullptr;
  int32_t dev_synced = 0;
};

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// HIP event pairs recorded around one kernel class (see oscar_kv_profile_*).
struct ProfClass {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  size_t used = 0;
};
constexpr size_t kProfMax = 8192;
constexpr int kMaxWinSplits = 48;   // bf16 window blocks per (sequence, kv head)
constexpr int kMinTilesPerWave = 3;  // INT2 tiles per wave below which splits are not added
constexpr int kSmallWinTokens = 64;   // window tokens per block when the launch is small
constexpr int kMergeOneTrip = 32;     // slots the head_dim-128 merge reads in one round trip

}  // namespace

struct oscar_kv {
  oscar_kv_config cfg{};
  int cap = 0;
  std::vector<Layer> layers;
  std::vector<void*> allocations;
  float* rk = nullptr;     // [L][D][D]
  float* rv = nullptr;     // [L][D][D]
  float* rvT = nullptr;    // [L][D][D] transposed
  uint16_t* rk3 = nullptr; // [L][3][D][D] bf16 pieces of R_K^T (R_K = sum of the three, transposed)
  uint16_t* rv3 = nullptr; // [L][3][D][D] the same for R_V
  float* qrot = nullptr;   // [B][Hq][D]
  float* qpub = nullptr;    // [B][Hkv][G][kQPub]
  float* partials = nullptr; // [B][Hq][kMaxSplits][D+2]
  unsigned* counters = nullptr; // [B][Hkv] blocks finished and producer steps done in the current
                                // decode launch (head_dim 128)
  float* vmax_pending = nullptr;  // [B][Hkv] V scale of the token a head_dim-128 decode step
                                  // appends, until its launch's merge folds it into smax
  size_t bytes = 0;
  int32_t forced_splits = 0;
  int32_t decode_impl = 0;   // oscar_kv_set_decode_impl
  int32_t mfma_waves = 4;
  int resident = 1024;       // matrix-core kernel blocks resident at once on the device
  int one_round = 0;         // one-round launches (test switch): r >= 3 always, with r blocks per
                             // (sequence, kv head); 0 or -1 never
  bool prof_on = false;
  ProfClass prof[3];
};

namespace {

int dev_alloc(oscar_kv* kv, void** p, size_t bytes) {
  if (bytes == 0) {
    *p = nullptr;
    return OSCAR_OK;
  }
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return fail(e == hipErrorOutOfMemory ? OSCAR_ERR_OUT_OF_MEMORY : OSCAR_ERR_HIP,
                std::string("hipMalloc(") + std::to_string(bytes) + "): " + hipGetErrorString(e));
  }
  kv->allocations.push_back(*p);
  kv->bytes += bytes;
  return OSCAR_OK;
}

void free_all(oscar_kv* kv) {
  for (void* p : kv->allocations) (void)hipFree(p);
  kv->allocations.clear();
  for (auto& pc : kv->prof) {
    for (auto& e : pc.ev) {
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
    pc.ev.clear();
    pc.used = 0;
  }
}

// Returns the slot recorded before a launch of class c, or -1 when not
// profiling.  The events only time work: they are created without the
// system-scope fence (cache write-back and invalidation) that a default event
// performs when it completes, which would slow the launches that follow.
long prof_begin(oscar_kv* kv, int c, hipStream_t s) {
  if (!kv->prof_on) return -1;
  ProfClass& pc = kv->prof[c];
  if (pc.used >= kProfMax) return -1;
  if (pc.used == pc.ev.size()) {
    hipEvent_t a, b;
    if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return -1;
    if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(a);
      return -1;
    }
    pc.ev.emplace_back(a, b);
  }
  if (hipEventRecord(pc.ev[pc.used].first, s) != hipSuccess) return -1;
  return (long)pc.used;
}

void prof_end(oscar_kv* kv, int c, long slot, hipStream_t s) {
  if (slot < 0) return;
  ProfClass& pc = kv->prof[c];
  if (hipEventRecord(pc.ev[(size_t)slot].second, s) == hipSuccess) pc.used = (size_t)slot + 1;
}

int validate_config(const oscar_kv_config* c) {
  if (!c) return fail(OSCAR_ERR_INVALID_ARG, "config is NULL");
  if (c->num_layers <= 0) return fail(OSCAR_ERR_INVALID_ARG, "num_layers must be > 0");
  if (c->max_batch <= 0) return fail(OSCAR_ERR_INVALID_ARG, "max_batch must be > 0");
  if (c->num_kv_heads <= 0 || c->num_q_heads <= 0)
    return fail(OSCAR_ERR_INVALID_ARG, "head counts must be > 0");
  if (c->num_q_heads % c->num_kv_heads != 0)
    return fail(OSCAR_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (c->num_q_heads / c->num_kv_heads > kMaxGq)
    return fail(OSCAR_ERR_UNSUPPORTED, "more than 16 query heads per kv head");
  if (c->group_size != kGroup) return fail(OSCAR_ERR_UNSUPPORTED, "group_size must be 128");
  if (c->head_dim != 128 && c->head_dim != 512)
    return fail(OSCAR_ERR_UNSUPPORTED, "head_dim must be 128 or 512");
  if (c->max_context <= 0) return fail(OSCAR_ERR_INVALID_ARG, "max_context must be > 0");
  if (c->sink_tokens < 0 || c->recent_tokens < 0)
    return fail(OSCAR_ERR_INVALID_ARG, "window sizes must be >= 0");
  if (c->codebook != OSCAR_CODEBOOK_UNIFORM && c->codebook != OSCAR_CODEBOOK_LLOYD_MAX)
    return fail(OSCAR_ERR_INVALID_ARG, "codebook must be 0 (uniform) or 1 (Lloyd-Max)");
  if (c->codebook == OSCAR_CODEBOOK_UNIFORM &&
      (!(c->k_clip > 0.0f && c->k_clip <= 1.0f) || !(c->v_clip > 0.0f && c->v_clip <= 1.0f)))
    return fail(OSCAR_ERR_INVALID_ARG, "clip ratios must be in (0, 1]");
  if (c->codebook == OSCAR_CODEBOOK_LLOYD_MAX && !(c->lm_ratio > 0.0f && c->lm_ratio <= 16.0f))
    return fail(OSCAR_ERR_INVALID_ARG, "lm_ratio must be in (0, 16]");
  // the caller may have stored any integer in the enum fields: read their
  // bits as int32 (reading an out-of-range value as the enum type is undefined)
  int32_t kd, vd;
  std::memcpy(&kd, &c->k_dtype, sizeof kd);
  std::memcpy(&vd, &c->v_dtype, sizeof vd);
  if ((kd != OSCAR_KV_INT2 && kd != OSCAR_KV_BF16) || (vd != OSCAR_KV_INT2 && vd != OSCAR_KV_BF16))
    return fail(OSCAR_ERR_INVALID_ARG, "unknown kv dtype");
  if ((long long)c->max_batch * c->num_q_heads > (1 << 30))
    return fail(OSCAR_ERR_INVALID_ARG, "batch x heads too large");
  if (c->absorb_v_rotation != 0 && c->absorb_v_rotation != 1)
    return fail(OSCAR_ERR_INVALID_ARG, "absorb_v_rotation must be 0 or 1");
  if (c->in_quant_hadamard != 0 && c->in_quant_hadamard != kGroup)
    return fail(OSCAR_ERR_INVALID_ARG, "in_quant_hadamard must be 0 or 128");
  return OSCAR_OK;
}

// The in-quant Hadamard folded into a rotation: every row r of R (rows of length D)
// becomes r H, H = the orthonormal Sylvester Walsh-Hadamard matrix of the given
// order on each order-wide block of the row, entry (i, j) = (-1)^popcount(i & j) /
// sqrt(order).  The butterflies (a, b) -> (a + b, a - b) run in fp64, the scale is
// applied once and the result is rounded to fp32 once.
void fold_hadamard(std::vector<float>& R, size_t rows, int D, int order) {
  const double scale = 1.0 / std::sqrt((double)order);
  std::vector<double> x(D);
  for (size_t r = 0; r < rows; ++r) {
    float* row = &R[r * D];
    for (int i = 0; i < D; ++i) x[i] = row[i];
    for (int base = 0; base < D; base += order)
      for (int h = 1; h < order; h <<= 1)
        for (int i = base; i < base + order; i += 2 * h)
          for (int j = i; j < i + h; ++j) {
            const double a = x[j], b = x[j + h];
            x[j] = a + b;
            x[j + h] = a - b;
          }
    for (int i = 0; i < D; ++i) row[i] = (float)(x[i] * scale);
  }
}

int alloc_plane(oscar_kv* kv, Plane* p, oscar_kv_dtype dt, bool is_v) {
  const auto& c = kv->cfg;
  const size_t BH = (size_t)c.max_batch * c.num_kv_heads;
  const size_t D = c.head_dim;
  int rc;
  if (dt == OSCAR_KV_BF16) {
    rc = dev_alloc(kv, (void**)&p->full, BH * kv->cap * D * 2);
    return rc;
  }
  if ((rc = dev_alloc(kv, (void**)&p->codes, BH * kv->cap * (D / 4)))) return rc;
  if ((rc = dev_alloc(kv, (void**)&p->meta, BH * kv->cap * (D / kGroup) * 4))) return rc;
  if ((rc = dev_alloc(kv, (void**)&p->sink, BH * c.sink_tokens * D * 2))) return rc;
  if ((rc = dev_alloc(kv, (void**)&p->ring, BH * c.recent_tokens * D * 2))) return rc;
  // stale metadata of unwritten positions must be finite: zero it once
  if (p->meta) HIP_TRY(hipMemset(p->meta, 0, BH * kv->cap * (D / kGroup) * 4));
  if (p->codes) HIP_TRY(hipMemset(p->codes, 0, BH * kv->cap * (D / 4)));
  if (is_v) {
    if ((rc = dev_alloc(kv, (void**)&p->smax, BH * sizeof(float)))) return rc;
    HIP_TRY(hipMemset(p->smax, 0, BH * sizeof(float)));
  }
  return OSCAR_OK;
}

PlaneDev plane_dev(const oscar_kv* kv, const Plane& p, bool is_v) {
  PlaneDev d{};
  d.codes = p.codes;
  d.meta = p.meta;
  d.sink = p.sink;
  d.ring = p.ring;
  d.full = p.full;
  d.smax = p.smax;
  d.lm = kv->cfg.codebook == OSCAR_CODEBOOK_LLOYD_MAX ? 1 : 0;
  d.clip = d.lm ? kv->cfg.lm_ratio : (is_v ? kv->cfg.v_clip : kv->cfg.k_clip);
  d.is_bf16 = (is_v ? kv->cfg.v_dtype : kv->cfg.k_dtype) == OSCAR_KV_BF16;
  d.tiled = is_v ? 1 : 0;
  return d;
}

// The planes of sequence `seq` alone, as those of a one-sequence batch: every
// pointer advanced by seq x Hkv (sequence, kv head) strides of its layout.
PlaneDev plane_dev_seq(const oscar_kv* kv, const Plane& p, bool is_v, int seq) {
  PlaneDev d = plane_dev(kv, p, is_v);
  const size_t bh = (size_t)seq * kv->cfg.num_kv_heads, D = kv->cfg.head_dim, cap = kv->cap;
  if (d.codes) d.codes += bh * cap * (D / 4);           // K rows and V tiles: cap * D / 4 bytes per (b, h)
  if (d.meta) d.meta += bh * (D / kGroup) * cap;
  if (d.sink) d.sink += bh * kv->cfg.sink_tokens * D;
  if (d.ring) d.ring += bh * kv->cfg.recent_tokens * D;
  if (d.full) d.full += bh * cap * D;
  if (d.smax) d.smax += bh;
  return d;
}

// Lengths of sequences [0, batch): the longest, the shortest, all equal.
struct BatchLens {
  int max = 0, min = 0;
  bool uniform = true;
};

BatchLens batch_lens(const Layer& L, int batch) {
  BatchLens r;
  r.max = r.min = L.lens[0];
  for (int b = 1; b < batch; ++b) {
    r.max = std::max(r.max, L.lens[b]);
    r.min = std::min(r.min, L.lens[b]);
  }
  r.uniform = r.max == r.min;
  return r;
}

// Writes lens[b] + add, b < batch, to the device copy (stream-ordered, the
// values travel as kernel arguments, nothing waits).
int upload_lens(Layer& L, int batch, int add, hipStream_t stream) {
  for (int first = 0; first < batch; first += kSetLensMax) {
    SetLensArgs a{};
    a.lens = L.dlens;
    a.first = first;
    a.n = std::min(kSetLensMax, batch - first);
    for (int i = 0; i < a.n; ++i) a.vals[i] = L.lens[first + i] + add;
    HIP_TRY(launch_set_lens(a, stream));
  }
  return OSCAR_OK;
}

void advance_lens(Layer& L, int batch, int add, bool synced) {
  for (int b = 0; b < batch; ++b) L.lens[b] += add;
  L.T = *std::max_element(L.lens.begin(), L.lens.end());
  L.dev_synced = synced ? batch : 0;
}

int check_layer(const oscar_kv* kv, int32_t layer) {
  if (!kv) return fail(OSCAR_ERR_INVALID_ARG, "handle is NULL");
  if (layer < 0 || layer >= kv->cfg.num_layers)
    return fail(OSCAR_ERR_INVALID_ARG, "layer " + std::to_string(layer) + " out of range");
  return OSCAR_OK;
}

int do_append(oscar_kv* kv, int32_t layer, const void* k, const void* v, int32_t batch, int32_t n_new,
              float* kdump, float* vdump, hipStream_t stream) {
  int rc = check_layer(kv, layer);
  if (rc) return rc;
  if (!k || !v) return fail(OSCAR_ERR_INVALID_ARG, "k/v pointer is NULL");
  if (batch <= 0 || batch > kv->cfg.max_batch)
    return fail(OSCAR_ERR_INVALID_ARG, "batch must be in [1, max_batch]");
  if (n_new <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_new must be > 0");
  Layer& L = kv->layers[layer];
  const BatchLens bl = batch_lens(L, batch);
  if ((long long)bl.max + n_new > kv->cfg.max_context)
    return fail(OSCAR_ERR_CAPACITY, "append of " + std::to_string(n_new) + " tokens to " +
                                        std::to_string(bl.max) + " exceeds max_context " +
                                        std::to_string(kv->cfg.max_context));
  // a ragged batch sizes the grid for the worst alignment of a sequence's
  // first new position (255 mod 256, so also 7 mod 8); each block then takes
  // its own sequence's positions from the device lengths
  const int T_old = bl.uniform ? bl.max : 255;
  const int groups = ((T_old + n_new - 1) >> 3) - (T_old >> 3) + 1;
  if (groups > 65535) return fail(OSCAR_ERR_INVALID_ARG, "n_new too large for one call (max 524272)");
  HIP_TRY(hipSetDevice(kv->cfg.device));
  if (!bl.uniform) {
    const int rc2 = upload_lens(L, batch, n_new, stream);
    if (rc2) return rc2;
  }
  AppendArgs a{};
  a.k = plane_dev(kv, L.k, false);
  a.v = plane_dev(kv, L.v, true);
  a.lens = bl.uniform ? nullptr : L.dlens;
  a.kin = static_cast<const uint16_t*>(k);
  a.vin = static_cast<const uint16_t*>(v);
  const size_t DD = (size_t)kv->cfg.head_dim * kv->cfg.head_dim;
  a.rk = kv->rk + layer * DD;
  a.rv = kv->rv + layer * DD;
  a.rk3 = kv->rk3 + layer * 3 * DD;
  a.rv3 = kv->rv3 + layer * 3 * DD;
  a.kdump = kdump;
  a.vdump = vdump;
  a.batch = batch;
  a.n_new = n_new;
  a.Hkv = kv->cfg.num_kv_heads;
  a.D = kv->cfg.head_dim;
  a.cap = kv->cap;
  a.N = kv->cfg.sink_tokens;
  a.M = kv->cfg.recent_tokens;
  a.T_old = T_old;
  a.T_new = T_old + n_new;
  const long ps = prof_begin(kv, 2, stream);
  if (n_new > 1)
    HIP_TRY(launch_append_prefill(a, stream));
  else
    HIP_TRY(launch_append(a, stream));
  prof_end(kv, 2, ps, stream);
  advance_lens(L, batch, n_new, !bl.uniform);
  return OSCAR_OK;
}

// Append n_new tokens to sequence `seq` alone: the append of a one-sequence
// batch on that sequence's planes.
int do_append_seq(oscar_kv* kv, int32_t layer, int32_t seq, const void* k, const void* v, int32_t n_new,
                  hipStream_t stream) {
  int rc = check_layer(kv, layer);
  if (rc) return rc;
  if (!k || !v) return fail(OSCAR_ERR_INVALID_ARG, "k/v pointer is NULL");
  if (seq < 0 || seq >= kv->cfg.max_batch) return fail(OSCAR_ERR_INVALID_ARG, "seq must be in [0, max_batch)");
  if (n_new <= 0) return fail(OSCAR_ERR_INVALID_ARG, "n_new must be > 0");
  Layer& L = kv->layers[layer];
  const int T0 = L.lens[seq];
  if ((long long)T0 + n_new > kv->cfg.max_context)
    return fail(OSCAR_ERR_CAPACITY, "append of " + std::to_string(n_new) + " tokens to " + std::to_string(T0) +
                                        " exceeds max_context " + std::to_string(kv->cfg.max_context));
  if (((T0 + n_new - 1) >> 3) - (T0 >> 3) + 1 > 65535)
    return fail(OSCAR_ERR_INVALID_ARG, "n_new too large for one call (max 524272)");
  HIP_TRY(hipSetDevice(kv->cfg.device));
  AppendArgs a{};
  a.k = plane_dev_seq(kv, L.k, false, seq);
  a.v = plane_dev_seq(kv, L.v, true, seq);
  a.kin = static_cast<const uint16_t*>(k);
  a.vin = static_cast<const uint16_t*>(v);
  const size_t DD = (size_t)kv->cfg.head_dim * kv->cfg.head_dim;
  a.rk = kv->rk + layer * DD;
  a.rv = kv->rv + layer * DD;
  a.rk3 = kv->rk3 + layer * 3 * DD;
  a.rv3 = kv->rv3 + layer * 3 * DD;
  a.batch = 1;
  a.n_new = n_new;
  a.Hkv = kv->cfg.num_kv_heads;
  a.D = kv->cfg.head_dim;
  a.cap = kv->cap;
  a.N = kv->cfg.sink_tokens;
  a.M = kv->cfg.recent_tokens;
  a.T_old = T0;
  a.T_new = T0 + n_new;
  const long ps = prof_begin(kv, 2, stream);
  if (n_new > 1)
    HIP_TRY(launch_append_prefill(a, stream));
  else
    HIP_TRY(launch_append(a, stream));
  prof_end(kv, 2, ps, stream);
  L.lens[seq] += n_new;
  L.T = std::max(L.T, L.lens[seq]);
  L.dev_synced = std::min(L.dev_synced, seq);
  return OSCAR_OK;
}

// Window tokens per window block (a multiple of 64).  At the 32k shape (320
// window tokens) 192 and 256 measured best: 66 and 65 us per launch against
// 70 us with 64 and 74 us with all 320 in one block.
constexpr int kWinTokens = 192;
constexpr int kWinTokensG2 = 128;       // 8 query heads per kv head (two head groups per window block)
// head_dim 512: bf16 window tokens per window block (512 measured 524 against
// 518 tokens/s for 256 at the wide-head 64k shape, 455 for 1024), INT2 blocks
// per launch
constexpr int kWideWinTokens = 512;
constexpr int kWideTargetBlocks = 1536;

// INT2 splits get equal shares of the range.  (Shares falling linearly from
// the first split to the last, for blocks dispatched later, measured slower
// with three tiles in flight per wave: 69.2 against 67.7 us per launch at the
// 32k shape with a fall of 0.4, 22.0 against 21.2 us at the 16k shape.)

// One-round launches (a test switch): a window chunk's cost as a fraction of
// a split's INT2 share (the INT2 shares of the blocks that carry one shrink by
// it).
constexpr float kOneRoundWinCost = 0.10f;

// INT2 splits per (sequence, kv head): as many blocks as are resident at once
// in total (measured at the 32k shape with two tiles in flight per wave: 6
// splits 82.4 us per launch against 87.9 with 12 and 83.5 with 4 or 5).
int auto_int2_splits(int BH, int ntiles, int waves, int resident) {
  int s = std::max(1, resident / std::max(1, BH));
  // at least kMinTilesPerWave tiles per wave: more splits only add merge slots
  s = std::min(s, std::max(1, ntiles / (std::max(1, waves) * kMinTilesPerWave)));
  return std::min(s, kMaxSplits - kMaxWinSplits);
}

SegPlan make_plan(int a0, int b0, int a1, int b1, int want_splits, int slot0) {
  SegPlan p{};
  p.a0 = a0;
  p.b0 = b0;
  p.a1 = a1;
  p.b1 = b1;
  const int len = std::max(0, b0 - a0) + std::max(0, b1 - a1);
  int chunk = (len + want_splits - 1) / want_splits;
  chunk = round_up(std::max(chunk, 1), kTile);
  p.chunk = chunk;
  p.splits = (len + chunk - 1) / chunk;
  p.slot0 = slot0;
  return p;
}

}  // namespace

extern "C" {

const char* oscar_last_error(void) { return g_last_error.c_str(); }

int oscar_kv_create(const oscar_kv_config* cfg, oscar_kv** out) {
  if (!out) return fail(OSCAR_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  int ndev = 0;
  HIP_TRY(hipGetDeviceCount(&ndev));
  if (cfg->device < 0 || cfg->device >= ndev) return fail(OSCAR_ERR_INVALID_ARG, "device out of range");
  HIP_TRY(hipSetDevice(cfg->device));
  oscar_kv* kv = new oscar_kv();
  kv->cfg = *cfg;
  kv->cfg.rot_k = nullptr;
  kv->cfg.rot_v = nullptr;
  kv->cap = round_up(cfg->max_context, kTile);
  kv->layers.resize(cfg->num_layers);
  const int L = cfg->num_layers, D = cfg->head_dim;
  const size_t DD = (size_t)D * D;
  auto bail = [&](int code) {
    free_all(kv);
    delete kv;
    return code;
  };
  for (int l = 0; l < L; ++l) {
    if ((rc = alloc_plane(kv, &kv->layers[l].k, cfg->k_dtype, false))) return bail(rc);
    if ((rc = alloc_plane(kv, &kv->layers[l].v, cfg->v_dtype, true))) return bail(rc);
    kv->layers[l].lens.assign(cfg->max_batch, 0);
    if ((rc = dev_alloc(kv, (void**)&kv->layers[l].dlens, (size_t)cfg->max_batch * sizeof(int)))) return bail(rc);
  }
  if ((rc = dev_alloc(kv, (void**)&kv->rk, L * DD * 4))) return bail(rc);
  if ((rc = dev_alloc(kv, (void**)&kv->rv, L * DD * 4))) return bail(rc);
  if ((rc = dev_alloc(kv, (void**)&kv->rvT, L * DD * 4))) return bail(rc);
  std::vector<float> rk(L * DD), rv(L * DD), rvT(L * DD);
  for (int l = 0; l < L; ++l)
    for (int e = 0; e < D; ++e)
      for (int d = 0; d < D; ++d) {
        const size_t i = l * DD + (size_t)e * D + d;
        rk[i] = cfg->rot_k ? cfg->rot_k[i] : (e == d ? 1.0f : 0.0f);
        rv[i] = cfg->rot_v ? cfg->rot_v[i] : (e == d ? 1.0f : 0.0f);
      }
  if (cfg->in_quant_hadamard) {
    fold_hadamard(rk, (size_t)L * D, D, cfg->in_quant_hadamard);
    fold_hadamard(rv, (size_t)L * D, D, cfg->in_quant_hadamard);
  }
  for (int l = 0; l < L; ++l)
    for (int e = 0; e < D; ++e)
      for (int d = 0; d < D; ++d) rvT[l * DD + (size_t)e * D + d] = rv[l * DD + (size_t)d * D + e];
  auto up = [&](void* dst, const void* src, size_t n) { return hipMemcpy(dst, src, n, hipMemcpyHostToDevice); };
  // bf16 pieces for the matrix-core prefill: R = R1 + R2 + R3 with R1 = bf16(R),
  // R2 = bf16(R - R1), R3 = bf16(R - R1 - R2) (each difference exact in fp32),
  // stored transposed ([column][row]) so that a lane's 8 consecutive rows are
  // one 16-byte load
  if ((rc = dev_alloc(kv, (void**)&kv->rk3, L * 3 * DD * 2))) return bail(rc);
  if ((rc = dev_alloc(kv, (void**)&kv->rv3, L * 3 * DD * 2))) return bail(rc);
  std::vector<uint16_t> rk3(L * 3 * DD), rv3(L * 3 * DD);
  for (int which = 0; which < 2; ++which) {
    const std::vector<float>& R = which ? rv : rk;
    std::vector<uint16_t>& out = which ? rv3 : rk3;
    for (size_t l = 0; l < L; ++l)
      for (int e = 0; e < D; ++e)
        for (int d = 0; d < D; ++d) {
          float r = R[l * DD + (size_t)e * D + d];
          for (int s = 0; s < 3; ++s) {
            const uint16_t p = f32_to_bf16(r);
            out[(l * 3 + s) * DD + (size_t)d * D + e] = p;
            r = r - bf16_to_f32(p);
          }
        }
  }
  if (up(kv->rk, rk.data(), L * DD * 4) != hipSuccess || up(kv->rv, rv.data(), L * DD * 4) != hipSuccess ||
      up(kv->rvT, rvT.data(), L * DD * 4) != hipSuccess || up(kv->rk3, rk3.data(), L * 3 * DD * 2) != hipSuccess ||
      up(kv->rv3, rv3.data(), L * 3 * DD * 2) != hipSuccess)
    return bail(fail(OSCAR_ERR_HIP, "copy of rotations failed"));
  const size_t B = cfg->max_batch, Hq = cfg->num_q_heads, Hkv = cfg->num_kv_heads;
  if ((rc = dev_alloc(kv, (void**)&kv->qrot, B * Hq * D * 4))) return bail(rc);
  // q records: one per 4 query heads (head_dim 128), one per 128-dim slice (head_dim 512)
  const size_t qrecs = std::max(std::max(Hkv, Hq / 4), D == 512 ? 4 * Hkv : (size_t)0);
  if ((rc = dev_alloc(kv, (void**)&kv->qpub, B * qrecs * kQPub * 4))) return bail(rc);
  if ((rc = dev_alloc(kv, (void**)&kv->partials, B * Hq * kMaxSplits * (D + 2) * 4))) return bail(rc);
  if ((rc = dev_alloc(kv, (void**)&kv->counters, B * Hkv * sizeof(unsigned)))) return bail(rc);
  if ((rc = dev_alloc(kv, (void**)&kv->vmax_pending, B * Hkv * sizeof(float)))) return bail(rc);
  if (hipMemset(kv->counters, 0, B * Hkv * sizeof(unsigned)) != hipSuccess ||
      hipMemset(kv->vmax_pending, 0, B * Hkv * sizeof(float)) != hipSuccess)
    return bail(fail(OSCAR_ERR_HIP, "clearing the decode counters failed"));
  if (hipDeviceSynchronize() != hipSuccess) return bail(fail(OSCAR_ERR_HIP, "device sync after create failed"));
  kv->resident = decode_mfma_resident_blocks(cfg->device, std::max(1, (int)(Hq / Hkv / 4)));
  *out = kv;
  g_last_error.clear();
  return OSCAR_OK;
}

int oscar_kv_destroy(oscar_kv* kv) {
  if (!kv) return OSCAR_OK;
  (void)hipSetDevice(kv->cfg.device);
  (void)hipDeviceSynchronize();
  free_all(kv);
  delete kv;
  return OSCAR_OK;
}

int oscar_kv_append(oscar_kv* kv, int32_t layer, const void* k, const void* v, int32_t batch,
                    int32_t n_new, hipStream_t stream) {
  return do_append(kv, layer, k, v, batch, n_new, nullptr, nullptr, stream);
}

int oscar_kv_append_dump(oscar_kv* kv, int32_t layer, const void* k, const void* v, int32_t batch,
                         int32_t n_new, float* k_rot, float* v_rot, hipStream_t stream) {
  if (!k_rot || !v_rot) return fail(OSCAR_ERR_INVALID_ARG, "dump pointer is NULL");
  return do_append(kv, layer, k, v, batch, n_new, k_rot, v_rot, stream);
}

int oscar_kv_append_seq(oscar_kv* kv, int32_t layer, int32_t seq, const void* k, const void* v, int32_t n_new,
                        hipStream_t stream) {
  return do_append_seq(kv, layer, seq, k, v, n_new, stream);
}

int oscar_kv_reset_seq(oscar_kv* kv, int32_t seq, hipStream_t stream) {
  if (!kv) return fail(OSCAR_ERR_INVALID_ARG, "handle is NULL");
  if (seq < 0 || seq >= kv->cfg.max_batch) return fail(OSCAR_ERR_INVALID_ARG, "seq must be in [0, max_batch)");
  HIP_TRY(hipSetDevice(kv->cfg.device));
  const int Hkv = kv->cfg.num_kv_heads;
  for (Layer& L : kv->layers) {
    // the running V scale maximum restarts with the sequence's new tokens
    if (L.v.smax) HIP_TRY(hipMemsetAsync(L.v.smax + (size_t)seq * Hkv, 0, Hkv * sizeof(float), stream));
    L.lens[seq] = 0;
    L.T = *std::max_element(L.lens.begin(), L.lens.end());
    L.dev_synced = std::min(L.dev_synced, seq);
  }
  return OSCAR_OK;
}

int oscar_kv_seq_length(const oscar_kv* kv, int32_t layer, int32_t seq, int32_t* tokens) {
  int rc = check_layer(kv, layer);
  if (rc) return rc;
  if (seq < 0 || seq >= kv->cfg.max_batch) return fail(OSCAR_ERR_INVALID_ARG, "seq must be in [0, max_batch)");
  if (!tokens) return fail(OSCAR_ERR_INVALID_ARG, "tokens is NULL");
  *tokens = kv->layers[layer].lens[seq];
  return OSCAR_OK;
}

}  // extern "C"

namespace {

bool fast_shape(const oscar_kv* kv) {
  const auto& c = kv->cfg;
  // the matrix-core kernel takes the codes as their integer values (uniform
  // codebook) and addresses one (sequence, kv head)'s code plane with 32-bit
  // buffer offsets: cap * 32 bytes must fit
  return kv->decode_impl != 1 && c.head_dim == 128 && c.codebook == OSCAR_CODEBOOK_UNIFORM &&
         (c.num_q_heads == 4 * c.num_kv_heads || c.num_q_heads == 8 * c.num_kv_heads) &&
         c.k_dtype == OSCAR_KV_INT2 && c.v_dtype == OSCAR_KV_INT2 && (long long)kv->cap * 32 <= INT32_MAX;
}

// head_dim 512 with at most 4 query heads per kv head, INT2 K, V INT2 or
// bf16, uniform codebook: the three-launch matrix-core path (32-bit buffer offsets: a (sequence,
// kv head)'s V plane, cap * 128 bytes INT2 or cap * 1024 bytes bf16, must fit)
bool wide_shape(const oscar_kv* kv) {
  const auto& c = kv->cfg;
  const int gq = c.num_q_heads / c.num_kv_heads;
  return kv->decode_impl != 1 && c.head_dim == 512 && c.codebook == OSCAR_CODEBOOK_UNIFORM &&
         (gq == 1 || gq == 2 || gq == 4) &&
         c.k_dtype == OSCAR_KV_INT2 && (long long)kv->cap * (c.v_dtype == OSCAR_KV_BF16 ? 1024 : 128) <= INT32_MAX;
}

int check_decode_args(const oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype,
                      float softmax_scale) {
  int rc = check_layer(kv, layer);
  if (rc) return rc;
  if (!q || !out) return fail(OSCAR_ERR_INVALID_ARG, "q/out pointer is NULL");
  if (out_dtype < 0 || out_dtype > 2) return fail(OSCAR_ERR_INVALID_ARG, "unknown out_dtype");
  if (!(softmax_scale == softmax_scale)) return fail(OSCAR_ERR_INVALID_ARG, "softmax_scale is NaN");
  return OSCAR_OK;
}

// Device memory a decode-attention call works in besides the cache and its
// inputs and outputs: the partial results (m, l, o') of its splits, the
// per-(sequence, kv head) counters of the head_dim-128 launch, the q records
// (written by that launch's producer blocks, or by the q rotation launch at
// head_dim 512), the rotated q of the general kernel.
// Either the handle's buffers (allocated at create) or the shared static
// array of the allocation-free call.
struct Scratch {
  bool use_static = false;
  unsigned char* base = nullptr;     // static array, this device's address
};

// Points the call's arguments at its working memory for `nslots` partial
// slots per (sequence, query head).  Static array: the fixed counter region,
// then q records, rotated q and partials carved for this call; CAPACITY when
// they do not fit.
int bind_scratch(oscar_kv* kv, const Scratch& sc, int batch, int nslots, DecodeArgs& da, CombineArgs& ca,
                 float** qrot = nullptr) {
  const auto& c = kv->cfg;
  if (!sc.use_static) {
    if (qrot) *qrot = kv->qrot;
    da.qrot = kv->qrot;
    da.qpub = kv->qpub;
    da.counters = kv->counters;
    da.partials = kv->partials;
    da.pstride = kMaxSplits;
    ca.partials = kv->partials;
    ca.pstride = kMaxSplits;
    return OSCAR_OK;
  }
  const size_t BH = (size_t)batch * c.num_kv_heads, BHq = (size_t)batch * c.num_q_heads, D = c.head_dim;
  const size_t qrecs = std::max(std::max((size_t)c.num_kv_heads, (size_t)c.num_q_heads / 4),
                                D == 512 ? 4 * (size_t)c.num_kv_heads : (size_t)0);
  auto up = [](size_t n) { return (n + 255) / 256 * 256; };
  const size_t off_qpub = kCounterBytes;
  const size_t off_qrot = off_qpub + up((size_t)batch * qrecs * kQPub * 4);
  const size_t off_part = off_qrot + up(BHq * D * 4);
  const size_t end = off_part + BHq * (size_t)nslots * (D + 2) * 4;
  if (BH * 4 > kCounterBytes || end > kStaticScratchBytes)
    return fail(OSCAR_ERR_CAPACITY, "the allocation-free decode call needs " + std::to_string(end) +
                                        " bytes of working memory for this batch and split plan; its static "
                                        "array holds " + std::to_string(kStaticScratchBytes) +
                                        " (use oscar_int2_decode_attn)");
  da.counters = reinterpret_cast<unsigned*>(sc.base);
  da.qpub = reinterpret_cast<float*>(sc.base + off_qpub);
  if (qrot) *qrot = reinterpret_cast<float*>(sc.base + off_qrot);
  da.qrot = reinterpret_cast<float*>(sc.base + off_qrot);
  da.partials = reinterpret_cast<float*>(sc.base + off_part);
  da.pstride = nslots;
  ca.partials = da.partials;
  ca.pstride = nslots;
  return OSCAR_OK;
}

// Enqueue decode attention of `layer` over T tokens.  With `app` set (matrix-
// core shapes only) the same launch also appends that one token, which is then
// the last of the T tokens.  dlens (ragged batch): the device token counts of
// the sequences, T then being the longest.
int launch_decode(oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype, int32_t batch,
                  float softmax_scale, int T, const AppendArgs* app, hipStream_t stream,
                  const Scratch& sc = Scratch(), const int* dlens = nullptr) {
  const Layer& L = kv->layers[layer];
  HIP_TRY(hipSetDevice(kv->cfg.device));
  const auto& c = kv->cfg;
  const int D = c.head_dim, Hq = c.num_q_heads, Hkv = c.num_kv_heads;
  const int N = c.sink_tokens, M = c.recent_tokens;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)D);
  const bool fast = fast_shape(kv);
  const size_t DD = (size_t)D * D;

  DecodeArgs da{};
  da.k = plane_dev(kv, L.k, false);
  da.v = plane_dev(kv, L.v, true);
  da.Hq = Hq;
  da.Hkv = Hkv;
  da.D = D;
  da.cap = kv->cap;
  da.N = N;
  da.M = M;
  da.T = T;
  da.Gq = Hq / Hkv;
  da.G = std::max(1, da.Gq / 4);
  da.q = static_cast<const uint16_t*>(q);
  da.rk = kv->rk + layer * DD;
  da.scale_log2 = scale * 1.4426950408889634f;
  da.app_blocks = app ? 2 : 0;
  if (app) da.app = *app;
  da.lens = dlens;
  CombineArgs ca{};
  ca.rvT = kv->rvT + layer * DD;
  ca.out = out;
  ca.out_dtype = out_dtype;
  ca.B = batch;
  ca.Hq = Hq;
  ca.Hkv = Hkv;
  ca.D = D;
  ca.absorb_v = c.absorb_v_rotation != 0;
  const int BH = batch * Hkv;

  // token sets: sink [0, min(N,T)), recent [max(N, T-M), T), INT2 [N, T-M)
  // (below N tokens the recent segment is empty: [T, T))
  const int sink_end = std::min(N, T);
  const int rec_begin = std::min(T, std::max(N, T - M));
  const int int2_lo = N, int2_hi = T - M;
  int rc = OSCAR_OK;
  const long pcall = sc.use_static ? -1 : prof_begin(kv, 1, stream);
  if (fast) {
    // bf16 window blocks and INT2 splits in one launch, merged by the last
    // block of each (sequence, kv head); q records (and a step's append) by a
    // prologue launch first, or by the launch's own blocks
    const int hp_len = sink_end + (T - rec_begin);
    SegPlan w{};
    if (hp_len > 0) {
      // window blocks are latency-bound (a memory round trip and three barriers
      // per 64-token pass): when the window is a large share of the tokens and
      // the launch leaves compute units idle (small batches, long windows), one
      // pass per block shortens the critical path.  Measured at batch 1, 16k
      // context, 2560 window tokens: 26.9 us per launch against 36.7 us.
      // two head groups double a window block's passes: shorter blocks
      const int wt = da.Gq == 8 ? kWinTokensG2 : kWinTokens;
      int want_w = (hp_len + wt - 1) / wt;
      const int int2_len = std::max(0, int2_hi - int2_lo);
      if ((long long)hp_len * 16 >= int2_len &&
          (long long)BH * ((hp_len + kSmallWinTokens - 1) / kSmallWinTokens) * 2 <= kv->resident)
        want_w = (hp_len + kSmallWinTokens - 1) / kSmallWinTokens;
      want_w = std::max(1, std::min(kMaxWinSplits, want_w));
      w = make_plan(0, sink_end, rec_begin, T, want_w, 0);
    }
    SegPlan p{};
    if (int2_hi > int2_lo) {
      const int ntiles = ((int2_hi - 1) >> 6) - (int2_lo >> 6) + 1;
      const int waves = kv->mfma_waves;
      int s = kv->forced_splits > 0 ? kv->forced_splits : auto_int2_splits(BH, ntiles, waves, kv->resident);
      s = std::max(1, std::min(s, std::min(ntiles, kMaxSplits - kMaxWinSplits)));
      const int tps = (ntiles + s - 1) / s;
      p.a0 = int2_lo;
      p.b0 = int2_hi;
      p.chunk = tps * kTile;
      p.splits = (ntiles + tps - 1) / tps;
    }
    // One round (test switch, R blocks per (sequence, kv head)): every block
    // is an INT2 split and the window chunks ride on splits 1 .. w (see
    // decode_mfma_kernel).  Never automatic: with three tiles in flight per
    // wave it measured 145.9 against 142.8 us per launch at the 128k shape,
    // and slower at the 32k shape too.
    const int R = kv->one_round;
    const bool one_round = R >= 3 && R <= kMaxOneRound;
    if (one_round) {
      p = SegPlan{};
      p.a0 = int2_lo;
      p.b0 = std::max(int2_lo, int2_hi);
      p.splits = R;
      w = hp_len > 0 ? make_plan(0, sink_end, rec_begin, T, R - 1, 0) : SegPlan{};
      // INT2 weight of each split: the window blocks start theirs after a
      // window chunk
      float wsum = 0.0f, wt[kMaxOneRound];
      for (int y = 0; y < R; ++y) {
        wt[y] = 1.0f;
        if (y >= 1 && y <= w.splits) wt[y] -= kOneRoundWinCost;
        wsum += wt[y];
      }
      float acc = 0.0f;
      for (int y = 0; y <= R; ++y) {
        da.share[y] = y == R ? 1.0f : acc / wsum;
        if (y < R) acc += wt[y];
      }
      da.one_round = 1;
    }
    // at most kMergeOneTrip slots per (sequence, kv head) when the windows
    // allow: the last block then merges in one memory round trip (measured at
    // the 16k shape, 14 window blocks instead of 40: 19.5 against 21.4 us)
    if (hp_len > 0 && !one_round && p.splits + w.splits > kMergeOneTrip && p.splits < kMergeOneTrip)
      w = make_plan(0, sink_end, rec_begin, T, kMergeOneTrip - p.splits, 0);
    p.slot0 = w.splits;      // window partials first, then the INT2 splits
    w.slot0 = 0;
    da.plan = p;
    da.win = w;
    // INT2 splits that fill the first wave of resident blocks go before the
    // window blocks
    da.win_blocks = w.splits;
    da.ring0 = M > 0 ? w.a1 % M : 0;
    da.int2_lead = std::max(0, std::min(p.splits, kv->resident / std::max(1, BH)));
    ca.nslots = p.splits + w.splits;
    if ((rc = bind_scratch(kv, sc, batch, ca.nslots, da, ca))) return rc;
    da.comb = ca;
    // One launch when every block of it is resident at once: each block
    // rotates its q itself and the window block that holds a step's token
    // appends it (a ring of at least a tile keeps that token out of the INT2
    // tiles the launch reads).  Measured at the 16k shape (256 blocks): 1400
    // against 1173 tokens/s with the prologue launch, which with the gap
    // between the two launches costs about 5 us per layer.  With more blocks
    // than are resident the window blocks run last and the rotation is
    // repeated in every block: at the 32k shape the one launch measured 73.4
    // us against 66.6 plus the prologue, no faster; the prologue launch then
    // writes q records (and appends) first.
    const long blocks = (long)BH * (one_round ? p.splits : p.splits + w.splits);
    const bool self = !one_round && kv->decode_impl != 2 && (!app || M >= kTile) &&
                      (kv->decode_impl == 3 || blocks <= kv->resident);
    da.self_rotate = self ? 1 : 0;
    if (self && app) {
      if (sc.use_static) return fail(OSCAR_ERR_INVALID_ARG, "the allocation-free call does not append");
      da.app.v.smax = kv->vmax_pending;
    }
    if (!self) {
      HIP_TRY(launch_decode_prologue(da, batch, stream));
      da.app_blocks = 0;
    }
    const long pk = sc.use_static ? -1 : prof_begin(kv, 0, stream);
    HIP_TRY(launch_decode_mfma(da, batch, kv->mfma_waves, stream));
    prof_end(kv, 0, pk, stream);
  } else if (wide_shape(kv)) {
    // q rotation records, then INT2 splits + bf16 window blocks, then the merge
    SegPlan w{};
    w.a0 = 0;
    w.b0 = sink_end;
    w.a1 = rec_begin;
    w.b1 = T;
    const int len0 = sink_end, len1 = T - rec_begin;
    int chunk = kWideWinTokens;
    auto nwin = [&](int ch) { return (len0 + ch - 1) / ch + (len1 + ch - 1) / ch; };
    while (nwin(chunk) > kMaxWinSplits) chunk *= 2;
    w.chunk = chunk;
    w.splits = nwin(chunk);
    w.slot0 = 0;
    SegPlan p{};
    if (int2_hi > int2_lo) {
      const int ntiles = ((int2_hi - 1) >> 6) - (int2_lo >> 6) + 1;
      int s = kv->forced_splits > 0 ? kv->forced_splits : std::max(1, kWideTargetBlocks / std::max(1, BH));
      s = std::max(1, std::min(s, std::min(ntiles, kMaxSplits - kMaxWinSplits)));
      p.a0 = int2_lo;
      p.b0 = int2_hi;
      p.splits = s;
    }
    p.slot0 = w.splits;
    da.plan = p;
    da.win = w;
    da.win_blocks = w.splits;
    da.ring0 = M > 0 ? rec_begin % M : 0;
    ca.nslots = p.splits + w.splits;
    if ((rc = bind_scratch(kv, sc, batch, ca.nslots, da, ca))) return rc;
    HIP_TRY(launch_wide_qrot(da, batch, stream));
    const long pk = sc.use_static ? -1 : prof_begin(kv, 0, stream);
    HIP_TRY(launch_decode_wide(da, batch, stream));
    prof_end(kv, 0, pk, stream);
    HIP_TRY(launch_combine(ca, stream));
  } else {
    int want = kv->forced_splits > 0 ? kv->forced_splits
                                     : std::max(1, std::min(64, 2048 / std::max(1, BH)));
    want = std::min(want, kMaxSplits);
    want = std::min(want, (T + kTile - 1) / kTile);
    da.plan = make_plan(0, T, 0, 0, want, 0);
    ca.nslots = da.plan.splits;
    float* qrot = nullptr;
    if ((rc = bind_scratch(kv, sc, batch, ca.nslots, da, ca, &qrot))) return rc;
    QRotArgs qa{};
    qa.q = static_cast<const uint16_t*>(q);
    qa.rk = kv->rk + layer * DD;
    qa.qrot = qrot;
    qa.B = batch;
    qa.Hq = Hq;
    qa.Hkv = Hkv;
    qa.D = D;
    qa.scale_log2 = da.scale_log2;
    HIP_TRY(launch_qrot(qa, stream));
    HIP_TRY(launch_decode_valu(da, batch, stream));
    HIP_TRY(launch_combine(ca, stream));
  }
  prof_end(kv, 1, pcall, stream);
  return OSCAR_OK;
}

// Decode attention of sequences [0, batch) over their current tokens: the
// uniform launch, or for a ragged batch the device lengths (uploaded first
// unless the device copy already holds them).
int decode_attn(oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype, int32_t batch,
                float softmax_scale, hipStream_t stream, Scratch sc) {
  int rc = check_decode_args(kv, layer, q, out, out_dtype, softmax_scale);
  if (rc) return rc;
  if (batch <= 0 || batch > kv->cfg.max_batch) return fail(OSCAR_ERR_INVALID_ARG, "batch must be in [1, max_batch]");
  Layer& L = kv->layers[layer];
  const BatchLens bl = batch_lens(L, batch);
  if (bl.min == 0) return fail(OSCAR_ERR_INVALID_ARG, "a sequence of the batch holds no tokens");
  HIP_TRY(hipSetDevice(kv->cfg.device));
  if (sc.use_static) HIP_TRY(static_scratch(kv->cfg.device, stream, &sc.base));
  if (bl.uniform) return launch_decode(kv, layer, q, out, out_dtype, batch, softmax_scale, bl.max, nullptr, stream, sc);
  if (L.dev_synced < batch) {
    if ((rc = upload_lens(L, batch, 0, stream))) return rc;
    L.dev_synced = batch;
  }
  return launch_decode(kv, layer, q, out, out_dtype, batch, softmax_scale, bl.max, nullptr, stream, sc, L.dlens);
}

}  // namespace

extern "C" {

int oscar_int2_decode_attn(oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype,
                           int32_t batch, float softmax_scale, hipStream_t stream) {
  return decode_attn(kv, layer, q, out, out_dtype, batch, softmax_scale, stream, Scratch());
}

int oscar_int2_decode_attn_noalloc(oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype,
                                   int32_t batch, float softmax_scale, hipStream_t stream) {
  Scratch sc;
  sc.use_static = true;
  return decode_attn(kv, layer, q, out, out_dtype, batch, softmax_scale, stream, sc);
}

int oscar_prefill_attn(oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype,
                       int32_t batch, int32_t n_q, float softmax_scale, hipStream_t stream) {
  int rc = check_decode_args(kv, layer, q, out, out_dtype, softmax_scale);
  if (rc) return rc;
  Layer& L = kv->layers[layer];
  const auto& c = kv->cfg;
  if (c.codebook != OSCAR_CODEBOOK_UNIFORM)
    return fail(OSCAR_ERR_UNSUPPORTED, "prefill attention needs the uniform codebook");
  // query rows per block: 64 at head_dim 128, 16 at 512
  const int rows = c.head_dim == 128 ? 64 : 16;
  if (rows % (c.num_q_heads / c.num_kv_heads) != 0)
    return fail(OSCAR_ERR_UNSUPPORTED, "prefill attention needs a power-of-two number of query heads per kv head, at "
                                       "most " + std::to_string(rows));
  if (batch <= 0 || batch > c.max_batch) return fail(OSCAR_ERR_INVALID_ARG, "batch must be in [1, max_batch]");
  const BatchLens bl = batch_lens(L, batch);
  if (n_q < 1 || n_q > bl.min)
    return fail(OSCAR_ERR_INVALID_ARG, "n_q must be in [1, tokens of every sequence of the batch]");
  HIP_TRY(hipSetDevice(c.device));
  if (!bl.uniform && L.dev_synced < batch) {
    if ((rc = upload_lens(L, batch, 0, stream))) return rc;
    L.dev_synced = batch;
  }
  const size_t DD = (size_t)c.head_dim * c.head_dim;
  PrefillAttnArgs a{};
  a.k = plane_dev(kv, L.k, false);
  a.v = plane_dev(kv, L.v, true);
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.out_dtype = out_dtype;
  a.rk = kv->rk + layer * DD;
  a.rvT = kv->rvT + layer * DD;
  a.absorb_v = c.absorb_v_rotation;
  a.B = batch;
  a.n = n_q;
  a.Hq = c.num_q_heads;
  a.Hkv = c.num_kv_heads;
  a.Gq = c.num_q_heads / c.num_kv_heads;
  a.cap = kv->cap;
  a.N = c.sink_tokens;
  a.M = c.recent_tokens;
  a.T = bl.max;
  a.D = c.head_dim;
  a.lens = bl.uniform ? nullptr : L.dlens;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  HIP_TRY(launch_prefill_attn(a, stream));
  return OSCAR_OK;
}

int oscar_kv_decode_step(oscar_kv* kv, int32_t layer, const void* k, const void* v, const void* q, void* out,
                         int32_t out_dtype, int32_t batch, float softmax_scale, hipStream_t stream) {
  int rc = check_decode_args(kv, layer, q, out, out_dtype, softmax_scale);
  if (rc) return rc;
  if (!k || !v) return fail(OSCAR_ERR_INVALID_ARG, "k/v pointer is NULL");
  if (batch <= 0 || batch > kv->cfg.max_batch) return fail(OSCAR_ERR_INVALID_ARG, "batch must be in [1, max_batch]");
  Layer& L = kv->layers[layer];
  const BatchLens bl = batch_lens(L, batch);
  if ((long long)bl.max + 1 > kv->cfg.max_context)
    return fail(OSCAR_ERR_CAPACITY, "decode step at " + std::to_string(bl.max) + " tokens exceeds max_context");
  if (!(fast_shape(kv) && kv->cfg.recent_tokens >= 1) && !wide_shape(kv)) {
    // separate launches: the appended token is not a bf16 window token here or
    // the shape has no fused kernel (head_dim 512 fuses the append with its q
    // rotation launch instead)
    rc = do_append(kv, layer, k, v, batch, 1, nullptr, nullptr, stream);
    if (rc) return rc;
    return decode_attn(kv, layer, q, out, out_dtype, batch, softmax_scale, stream, Scratch());
  }
  HIP_TRY(hipSetDevice(kv->cfg.device));
  if (!bl.uniform && (rc = upload_lens(L, batch, 1, stream))) return rc;
  AppendArgs a{};
  a.k = plane_dev(kv, L.k, false);
  a.v = plane_dev(kv, L.v, true);
  a.kin = static_cast<const uint16_t*>(k);
  a.vin = static_cast<const uint16_t*>(v);
  const size_t DD = (size_t)kv->cfg.head_dim * kv->cfg.head_dim;
  a.rk = kv->rk + layer * DD;
  a.rv = kv->rv + layer * DD;
  a.batch = batch;
  a.n_new = 1;
  a.Hkv = kv->cfg.num_kv_heads;
  a.D = kv->cfg.head_dim;
  a.cap = kv->cap;
  a.N = kv->cfg.sink_tokens;
  a.M = kv->cfg.recent_tokens;
  a.T_old = bl.max;
  a.T_new = bl.max + 1;
  a.lens = bl.uniform ? nullptr : L.dlens;
  rc = launch_decode(kv, layer, q, out, out_dtype, batch, softmax_scale, bl.max + 1, &a, stream, Scratch(), a.lens);
  if (rc) return rc;
  advance_lens(L, batch, 1, !bl.uniform);
  return OSCAR_OK;
}

int oscar_kv_profile_enable(oscar_kv* kv, int32_t enable) {
  if (!kv) return fail(OSCAR_ERR_INVALID_ARG, "handle is NULL");
  for (auto& pc : kv->prof) pc.used = 0;
  kv->prof_on = enable != 0;
  return OSCAR_OK;
}

int oscar_kv_profile_read(oscar_kv* kv, int32_t kernel_class, double* total_ms, int64_t* launches) {
  if (!kv || !total_ms || !launches) return fail(OSCAR_ERR_INVALID_ARG, "NULL argument");
  if (kernel_class < 0 || kernel_class > 2) return fail(OSCAR_ERR_INVALID_ARG, "kernel_class must be 0..2");
  HIP_TRY(hipSetDevice(kv->cfg.device));
  ProfClass& pc = kv->prof[kernel_class];
  double sum = 0.0;
  for (size_t i = 0; i < pc.used; ++i) {
    HIP_TRY(hipEventSynchronize(pc.ev[i].second));
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, pc.ev[i].first, pc.ev[i].second));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)pc.used;
  return OSCAR_OK;
}

int oscar_kv_length(const oscar_kv* kv, int32_t layer, int32_t* tokens) {
  int rc = check_layer(kv, layer);
  if (rc) return rc;
  if (!tokens) return fail(OSCAR_ERR_INVALID_ARG, "tokens is NULL");
  *tokens = kv->layers[layer].T;
  return OSCAR_OK;
}

int oscar_kv_device_bytes(const oscar_kv* kv, size_t* bytes) {
  if (!kv || !bytes) return fail(OSCAR_ERR_INVALID_ARG, "NULL argument");
  *bytes = kv->bytes;
  return OSCAR_OK;
}

int oscar_kv_set_num_splits(oscar_kv* kv, int32_t num_splits) {
  if (!kv) return fail(OSCAR_ERR_INVALID_ARG, "handle is NULL");
  if (num_splits < 0 || num_splits > kMaxSplits - kMaxWinSplits)
    return fail(OSCAR_ERR_INVALID_ARG, "num_splits must be in [0, 224]");
  kv->forced_splits = num_splits;
  return OSCAR_OK;
}

int oscar_kv_set_one_round(oscar_kv* kv, int32_t blocks) {
  if (!kv) return fail(OSCAR_ERR_INVALID_ARG, "handle is NULL");
  if (!(blocks == 0 || blocks == -1 || (blocks >= 3 && blocks <= kMaxOneRound)))
    return fail(OSCAR_ERR_INVALID_ARG, "blocks must be 0, -1 or in [3, 16]");
  kv->one_round = blocks;
  return OSCAR_OK;
}

int oscar_kv_set_decode_impl(oscar_kv* kv, int32_t impl) {
  if (!kv) return fail(OSCAR_ERR_INVALID_ARG, "handle is NULL");
  if (impl < 0 || impl > 3) return fail(OSCAR_ERR_INVALID_ARG, "impl must be 0, 1, 2 or 3");
  kv->decode_impl = impl;
  return OSCAR_OK;
}

int oscar_kv_export(oscar_kv* kv, int32_t layer, int32_t which, void* host_codes, void* host_meta,
                    void* host_sink, void* host_ring) {
  int rc = check_layer(kv, layer);
  if (rc) return rc;
  if (which != 0 && which != 1) return fail(OSCAR_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V)");
  HIP_TRY(hipSetDevice(kv->cfg.device));
  HIP_TRY(hipDeviceSynchronize());
  const auto& c = kv->cfg;
  const Layer& L = kv->layers[layer];
  const Plane& p = which ? L.v : L.k;
  const bool bf16 = (which ? c.v_dtype : c.k_dtype) == OSCAR_KV_BF16;
  const int BH = c.max_batch * c.num_kv_heads, D = c.head_dim, T = L.T, cap = kv->cap;
  if (bf16) {
    if (host_codes && T > 0)
      HIP_TRY(hipMemcpy2D(host_codes, (size_t)T * D * 2, p.full, (size_t)cap * D * 2, (size_t)T * D * 2, BH,
                          hipMemcpyDeviceToHost));
    return OSCAR_OK;
  }
  if (host_codes && T > 0) {
    // both planes are stored tiled; the export is canonical [BH][T][D/4]
    uint8_t* tmp = nullptr;
    HIP_TRY(hipMalloc(&tmp, (size_t)BH * T * (D / 4)));
    hipError_t e = launch_export_codes(p.codes, tmp, BH, cap, T, D, which, nullptr);
    if (e == hipSuccess) e = hipMemcpy(host_codes, tmp, (size_t)BH * T * (D / 4), hipMemcpyDeviceToHost);
    (void)hipFree(tmp);
    HIP_TRY(e);
  }
  if (host_meta && T > 0) {
    // stored group-major [BH][D/128][cap]; the export is [BH][T][D/128]
    const int G = D / kGroup;
    std::vector<uint32_t> tmp((size_t)BH * G * T);
    HIP_TRY(hipMemcpy2D(tmp.data(), (size_t)T * 4, p.meta, (size_t)cap * 4, (size_t)T * 4, (size_t)BH * G,
                        hipMemcpyDeviceToHost));
    uint32_t* dst = static_cast<uint32_t*>(host_meta);
    for (size_t bh = 0; bh < (size_t)BH; ++bh)
      for (int g = 0; g < G; ++g)
        for (int t = 0; t < T; ++t) dst[(bh * T + t) * G + g] = tmp[(bh * G + g) * T + t];
  }
  if (host_sink && c.sink_tokens > 0)
    HIP_TRY(hipMemcpy(host_sink, p.sink, (size_t)BH * c.sink_tokens * D * 2, hipMemcpyDeviceToHost));
  if (host_ring && c.recent_tokens > 0)
    HIP_TRY(hipMemcpy(host_ring, p.ring, (size_t)BH * c.recent_tokens * D * 2, hipMemcpyDeviceToHost));
  return OSCAR_OK;
}

int oscar_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0) return fail(OSCAR_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (bytes > 0 && (!src || !dst)) return fail(OSCAR_ERR_INVALID_ARG, "NULL pointer");
  HIP_TRY(launch_stream_copy(src, dst, bytes, stream));
  return OSCAR_OK;
}

int oscar_stream_read(const void* src, size_t bytes, void* xor_out, hipStream_t stream) {
  if (bytes % 16 != 0) return fail(OSCAR_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (!xor_out || (bytes > 0 && !src)) return fail(OSCAR_ERR_INVALID_ARG, "NULL pointer");
  HIP_TRY(launch_stream_read(src, bytes, static_cast<unsigned*>(xor_out), stream));
  return OSCAR_OK;
}

int oscar_quantize_rows(const float* x, int32_t rows, int32_t D, int32_t G, float clip, void* codes,
                        void* meta, hipStream_t stream) {
  if (rows < 0) return fail(OSCAR_ERR_INVALID_ARG, "rows must be >= 0");
  if (G != kGroup) return fail(OSCAR_ERR_UNSUPPORTED, "group size must be 128");
  if (D != 128 && D != 512) return fail(OSCAR_ERR_UNSUPPORTED, "D must be 128 or 512");
  if (!(clip > 0.0f && clip <= 1.0f)) return fail(OSCAR_ERR_INVALID_ARG, "clip must be in (0, 1]");
  if (rows > 0 && (!x || !codes || !meta)) return fail(OSCAR_ERR_INVALID_ARG, "NULL pointer");
  HIP_TRY(launch_quantize_rows(x, rows, D, clip, 0, static_cast<uint8_t*>(codes), static_cast<uint32_t*>(meta),
                               stream));
  return OSCAR_OK;
}

int oscar_quantize_rows_lloyd_max(const float* x, int32_t rows, int32_t D, int32_t G, float ratio, void* codes,
                                  void* meta, hipStream_t stream) {
  if (rows < 0) return fail(OSCAR_ERR_INVALID_ARG, "rows must be >= 0");
  if (G != kGroup) return fail(OSCAR_ERR_UNSUPPORTED, "group size must be 128");
  if (D != 128 && D != 512) return fail(OSCAR_ERR_UNSUPPORTED, "D must be 128 or 512");
  if (!(ratio > 0.0f && ratio <= 16.0f)) return fail(OSCAR_ERR_INVALID_ARG, "ratio must be in (0, 16]");
  if (rows > 0 && (!x || !codes || !meta)) return fail(OSCAR_ERR_INVALID_ARG, "NULL pointer");
  HIP_TRY(launch_quantize_rows(x, rows, D, ratio, 1, static_cast<uint8_t*>(codes), static_cast<uint32_t*>(meta),
                               stream));
  return OSCAR_OK;
}

}  // extern "C"
