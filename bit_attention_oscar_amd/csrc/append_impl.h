// Device code of the append path, shared by the append kernel and by the fused
// decode-step launch (which appends the new token in the same launch as the
// attention over the cache).
//
// Method (web pages on OSCAR): rotation of post-RoPE K and V by one orthogonal
// head_dim x head_dim matrix per layer ("OSCAR-LLAMACPP-Qwen3-4B-Thinking-2507-
// INT2-KV", "Files" note; "OSCAR-RotationZoo", "File format"); clip before
// quantization (Qwen3-4B card, "Run" env-var table; K 0.96 / V 0.92 in the
// RotationZoo card, "How to use" step 2); INT2 with group 128 along head_dim
// (RotationZoo card, same flags); bf16 sink and recent window (Qwen3-4B card,
// "Run" table; "OSCAR: 2-bit KV Cache Quantization for SGLang and llama.cpp",
// "What OSCAR compresses").
//
// Every file including this header is built with -ffp-contract=off and
// correctly rounded fp32 division: the quantizer performs exactly one IEEE
// rounding per operation.
#pragma once
#include "common.h"

namespace oscar {

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

struct GroupQ {
  float sf, zf;      // stored scale / zero widened to fp32
  uint32_t packed;   // fp16 scale bits | fp16 zero bits << 16
};

// Keeps a value as a materialised fp32 register: stops the compiler from
// folding the product into a mixed-precision fma that rounds straight to fp16
// (one rounding of the exact product instead of fp32 then fp16).
__device__ inline float as_f32(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// hi = r*max, lo = r*min, s = (hi - lo)/3; fp16 RNE of s and lo.
__device__ inline GroupQ group_params(float mx, float mn, float r) {
  const float hi = as_f32(r * mx);
  const float lo = as_f32(r * mn);
  const float s = as_f32((hi - lo) / 3.0f);
  const _Float16 s16 = (_Float16)s;
  const _Float16 z16 = (_Float16)lo;
  GroupQ g;
  g.sf = (float)s16;
  g.zf = (float)z16;
  g.packed = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
             ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
  return g;
}

// c = clamp(rint((x - z)/s), 0, 3), round half to even; 0 when s == 0.
__device__ inline uint32_t quant_code(float x, const GroupQ& g) {
  if (g.sf == 0.0f) return 0u;
  float t = (x - g.zf) / g.sf;
  t = __builtin_rintf(t);
  t = fminf(fmaxf(t, 0.0f), 3.0f);
  return (uint32_t)t;
}

// quant_code with the division replaced where that provably changes nothing:
// inv = v_rcp_f32(s) (1 ulp), so qa = (x - z) * inv is within 2^-20 of the
// exact quotient Q = (x - z) / s for |Q| < 4, and the correctly rounded
// quotient q is within 2^-23 of Q.  If qa is at least 2^-17 away from 0.5,
// 1.5 and 2.5, Q and q lie strictly on the side of that half-integer where qa
// lies, so rint(q) = rint(qa); otherwise (rare) the correctly rounded division
// decides.  Outside (0, 3) the clamp gives the same code either way.
__device__ inline uint32_t quant_code_fast(float x, const GroupQ& g, float inv) {
  if (g.sf == 0.0f) return 0u;
  const float d = x - g.zf;
  const float qa = d * inv;
  const float fr = qa - __builtin_floorf(qa);
  float t;
  if (qa > 0.0f && qa < 3.0f && __builtin_fabsf(fr - 0.5f) < 0x1p-17f)
    t = __builtin_rintf(d / g.sf);
  else
    t = __builtin_rintf(qa);
  t = fminf(fmaxf(t, 0.0f), 3.0f);
  return (uint32_t)t;
}

// Lloyd-Max codebook (levels and threshold in common.h).  A group's
// statistics are sums in one fixed pairwise order: element i with i + 64,
// then with i + 32, ..., then with i + 1, each add rounded once, so that
// every layout of the group's 128 values gives the same bits.

// Sum of a group held two values per lane (dims lane and lane + 64): the first
// add pairs i with i + 64 in-lane; lanes l and l ^ k then add the same two
// values, so every lane ends with the same sum.
__device__ inline float group_sum128(float a, float b) {
  float s = as_f32(a + b);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s = as_f32(s + __shfl_xor(s, o));
  return s;
}

// mean = sum / 128, variance = sum of squared deviations / 128 (division by a
// power of two: exact), s = ratio * sqrt(variance) with the correctly rounded
// square root; fp16 RNE of s and the mean.
__device__ inline GroupQ lm_group_params(float mean, float sumsq, float ratio) {
  const float var = as_f32(sumsq * 0.0078125f);
  const float s = as_f32(ratio * as_f32(__builtin_sqrtf(var)));
  const _Float16 s16 = (_Float16)s;
  const _Float16 z16 = (_Float16)mean;
  GroupQ g;
  g.sf = (float)s16;
  g.zf = (float)z16;
  g.packed = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
             ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
  return g;
}

// the level nearest to x among z + s * level(c): u = (x - z) / s (correctly
// rounded), c = [u >= -tau] + [u >= 0] + [u >= tau]; 0 when s == 0.
__device__ inline uint32_t lm_code(float x, const GroupQ& g) {
  if (g.sf == 0.0f) return 0u;
  const float u = as_f32(x - g.zf) / g.sf;
  return (uint32_t)(u >= -kLmThreshold) + (uint32_t)(u >= 0.0f) + (uint32_t)(u >= kLmThreshold);
}

// Lloyd-Max parameters of a group held two per lane (dims lane, lane + 64).
__device__ inline GroupQ lm_group_wave(float x0, float x1, float ratio) {
  const float mean = as_f32(group_sum128(x0, x1) * 0.0078125f);
  const float d0 = as_f32(x0 - mean), d1 = as_f32(x1 - mean);
  return lm_group_params(mean, group_sum128(as_f32(d0 * d0), as_f32(d1 * d1)), ratio);
}

// Canonical packing through lane shuffles: lane l holds the code of dim
// l + 64 i; word w (dims 16w..16w+15) is OR-reduced over the 16 lanes
// 16 (w % 4) .. + 15 of element i = w / 4 and stored by its first lane at
// word_addr(w).
template <int PER, class WordAddr>
__device__ inline void store_canonical(const uint32_t* code, int lane, WordAddr word_addr) {
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    uint32_t v = code[i] << (2 * (lane & 15));
    v |= __shfl_xor(v, 1);
    v |= __shfl_xor(v, 2);
    v |= __shfl_xor(v, 4);
    v |= __shfl_xor(v, 8);
    if ((lane & 15) == 0) *word_addr(4 * i + (lane >> 4)) = v;
  }
}

// Rotation of NT token rows held in xs[NT][D] (fp32) by R (fp32 [D][D]):
// wave w accumulates x[e] * R[e][d] over e in [w D/WAVES, (w+1) D/WAVES),
// e ascending, with fused multiply-adds, into part[w][tk][d].  The caller
// synchronises, then reads rot_sum(), which adds the partials in a fixed order
// and maps -0 to +0: every user of this routine gets identical bits.
template <int D, int WAVES, int NT>
__device__ inline void rotate_rows(const float* xs, const float* R, float* part, int ntok) {
  constexpr int PER = D / 64;
  constexpr int EW = D / WAVES;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float acc[NT][PER];
#pragma unroll
  for (int tk = 0; tk < NT; ++tk)
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[tk][i] = 0.0f;
  const float* Rw = R + (size_t)(wave * EW) * D + lane;
#pragma unroll 8
  for (int e = 0; e < EW; ++e) {
    float r[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) r[i] = Rw[(size_t)e * D + 64 * i];
#pragma unroll
    for (int tk = 0; tk < NT; ++tk) {
      const float x = xs[tk * D + wave * EW + e];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[tk][i] = __builtin_fmaf(x, r[i], acc[tk][i]);
    }
  }
#pragma unroll
  for (int tk = 0; tk < NT; ++tk)
#pragma unroll
    for (int i = 0; i < PER; ++i) part[(wave * NT + tk) * D + lane + 64 * i] = acc[tk][i];
  (void)ntok;
}

// The same rotation with this lane's rows of R loaded up front into
// registers (head_dim 128: 32 rows of e, dims lane and lane + 64), so that a
// block can issue them together with its other loads: one memory round trip
// instead of one per chunk of e.  Identical arithmetic and bits.
template <int D, int WAVES>
struct RRows {
  static constexpr int EW = D / WAVES, PER = D / 64;
  float r[EW][PER];
};

template <int D, int WAVES>
__device__ inline RRows<D, WAVES> load_r_rows(const float* R) {
  RRows<D, WAVES> rr;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* Rw = R + (size_t)(wave * RRows<D, WAVES>::EW) * D + lane;
#pragma unroll
  for (int e = 0; e < RRows<D, WAVES>::EW; ++e)
#pragma unroll
    for (int i = 0; i < RRows<D, WAVES>::PER; ++i) rr.r[e][i] = Rw[(size_t)e * D + 64 * i];
  return rr;
}

template <int D, int WAVES, int NT>
__device__ inline void rotate_rows_regs(const float* xs, const RRows<D, WAVES>& rr, float* part) {
  constexpr int PER = D / 64, EW = D / WAVES;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float acc[NT][PER];
#pragma unroll
  for (int tk = 0; tk < NT; ++tk)
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[tk][i] = 0.0f;
#pragma unroll
  for (int e = 0; e < EW; ++e)
#pragma unroll
    for (int tk = 0; tk < NT; ++tk) {
      const float x = xs[tk * D + wave * EW + e];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[tk][i] = __builtin_fmaf(x, rr.r[e][i], acc[tk][i]);
    }
#pragma unroll
  for (int tk = 0; tk < NT; ++tk)
#pragma unroll
    for (int i = 0; i < PER; ++i) part[(wave * NT + tk) * D + lane + 64 * i] = acc[tk][i];
}

template <int D, int WAVES, int NT>
__device__ inline float rot_sum(const float* part, int tk, int d) {
  float v = part[tk * D + d];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) v = v + part[(w * NT + tk) * D + d];
  return v + 0.0f;   // -0 -> +0
}

// A bf16 window value (sink or ring row).  CW: a device-scope store, visible
// to blocks on every XCD once it completes, for a launch whose other blocks
// read the row after this one signals them.
template <bool CW>
__device__ inline void put_window(uint16_t* p, float x) {
  if constexpr (CW)
    __hip_atomic_store(p, f32_to_bf16(x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = f32_to_bf16(x);
}

// Wave 0's part of an append, after the rotation: for each token, the rotated
// row from the partial sums in part (rot_sum), the window rows, the group
// statistics, codes and scale|zero words.  vbyte: with one token, the V code
// bytes of the lane's dims, loaded beforehand.
template <int D, int WAVES, int NT, bool LM, bool CW>
__device__ inline void append_tail(const AppendArgs& a, int bh, bool isv, int t_lo, int ntok, int T_old, int T_new,
                                   const float* part, const uint8_t (&vbyte)[D / 64]) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const PlaneDev P = isv ? a.v : a.k;
  float* dump = isv ? a.vdump : a.kdump;
#pragma unroll
  for (int tk = 0; tk < NT; ++tk) {
    if (tk >= ntok) break;
    const int t = t_lo + tk;
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = rot_sum<D, WAVES, NT>(part, tk, lane + 64 * i);
    if (dump) {
      const size_t base = (((size_t)b * a.n_new + (t - T_old)) * a.Hkv + h) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) dump[base + lane + 64 * i] = x[i];
    }
    if (P.is_bf16) {
      const size_t base = row_offset(bh, a.cap, t, D);
#pragma unroll
      for (int i = 0; i < PER; ++i) P.full[base + lane + 64 * i] = f32_to_bf16(x[i]);
      continue;
    }
    if (t < a.N) {
      const size_t base = row_offset(bh, a.N, t, D);
#pragma unroll
      for (int i = 0; i < PER; ++i) put_window<CW>(P.sink + base + lane + 64 * i, x[i]);
    }
    if (a.M > 0 && t >= a.N && t >= T_new - a.M) {
      const size_t base = row_offset(bh, a.M, t % a.M, D);
#pragma unroll
      for (int i = 0; i < PER; ++i) put_window<CW>(P.ring + base + lane + 64 * i, x[i]);
    }
    uint32_t code[PER];
#pragma unroll
    for (int g = 0; g < D / kGroup; ++g) {
      // group g = dims [128 g, 128 g + 128) = elements 2g, 2g+1 of every lane
      GroupQ q;
      if constexpr (LM) {
        q = lm_group_wave(x[2 * g], x[2 * g + 1], P.clip);
        code[2 * g] = lm_code(x[2 * g], q);
        code[2 * g + 1] = lm_code(x[2 * g + 1], q);
      } else {
        const float mx = wave_max(fmaxf(x[2 * g], x[2 * g + 1]));
        const float mn = wave_min(fminf(x[2 * g], x[2 * g + 1]));
        q = group_params(mx, mn, P.clip);
        code[2 * g] = quant_code(x[2 * g], q);
        code[2 * g + 1] = quant_code(x[2 * g + 1], q);
      }
      if (lane == 0) {
        P.meta[meta_index(bh, a.cap, t, g, D)] = q.packed;
        if (P.smax) atomicMax(reinterpret_cast<unsigned int*>(P.smax + bh), __float_as_uint(q.sf));
      }
    }
    if (!P.tiled) {
      store_canonical<PER>(code, lane, [&](int w) {
        return reinterpret_cast<uint32_t*>(P.codes + kcode_byte(bh, a.cap, t, 4 * w, D));
      });
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int bit;
        const size_t off = vcode_byte(bh, a.cap, t, lane + 64 * i, D, &bit);
        const uint8_t old = NT == 1 ? vbyte[i] : P.codes[off];
        P.codes[off] = (uint8_t)((old & ~(3u << bit)) | (code[i] << bit));
      }
    }
  }
}

// Append of tokens [t_lo, t_hi) (at most NT, all in one 8-token group) of one
// (sequence, kv head) to plane K (isv = false) or V.  Block = 64 * WAVES
// threads; xs holds NT*D floats and part WAVES*NT*D floats of shared memory.
// Wave 0's lane l owns dims l + 64 i, so it also owns the V tile bytes of those
// dims for every token of the group (tiled-layout bytes are shared only among
// tokens of one group of 8 at one dim, and one block handles the whole group).
// With one token (NT = 1) those bytes are loaded together with the inputs, so
// that their rewrite needs no second memory round trip.  CW: the window rows
// are written with device-scope stores (put_window).
template <int D, int WAVES, int NT, bool LM = false, bool CW = false>
__device__ inline void append_block(const AppendArgs& a, int bh, bool isv, int t_lo, int t_hi, int T_old, int T_new,
                                    float* xs, float* part) {
  constexpr int PER = D / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const PlaneDev P = isv ? a.v : a.k;
  const uint16_t* in = isv ? a.vin : a.kin;
  const float* R = isv ? a.rv : a.rk;
  const int ntok = t_hi - t_lo;
  uint8_t vbyte[PER];                  // NT = 1, tiled plane: the code bytes of the token's dims
#pragma unroll
  for (int i = 0; i < PER; ++i) vbyte[i] = 0;
  if constexpr (NT == 1) {
    if (wave == 0 && ntok > 0 && !P.is_bf16 && P.tiled) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int bit;
        vbyte[i] = P.codes[vcode_byte(bh, a.cap, t_lo, lane + 64 * i, D, &bit)];
      }
    }
  }

  auto load_inputs = [&]() {
    for (int i = tid; i < NT * D; i += 64 * WAVES) {
      const int tk = i / D, d = i - (i / D) * D;
      float v = 0.0f;
      if (tk < ntok) {
        const int t = t_lo + tk;
        const size_t idx = (((size_t)b * a.n_new + (t - T_old)) * a.Hkv + h) * D + d;
        v = bf16_to_f32(in[idx]);
      }
      xs[i] = v;
    }
  };
  if constexpr (D == 128 && WAVES == 4) {
    // R rows and inputs in one round trip
    const RRows<D, WAVES> rr = load_r_rows<D, WAVES>(R);
    load_inputs();
    __syncthreads();
    rotate_rows_regs<D, WAVES, NT>(xs, rr, part);
  } else {
    load_inputs();
    __syncthreads();
    rotate_rows<D, WAVES, NT>(xs, R, part, ntok);
  }
  __syncthreads();
  if (wave != 0) return;
  append_tail<D, WAVES, NT, LM, CW>(a, bh, isv, t_lo, ntok, T_old, T_new, part, vbyte);
}

// One-token append at head_dim 128 (4 waves) in two steps, for a block that
// issues other loads between them: append_one_loads issues every load the
// append needs (this lane's R rows as load_r_rows takes them, the token's
// input value in threads < 128, wave 0's V code bytes); append_one_finish does
// the rest exactly as append_block<128, 4, 1> does (same rotation, same bits).
struct AppendOneLoads {
  RRows<128, 4> rr;
  float x;
  uint8_t vbyte[2];
};

__device__ __forceinline__ AppendOneLoads append_one_loads(const AppendArgs& a, int bh, bool isv, int t, int T_old) {
  constexpr int D = 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const PlaneDev P = isv ? a.v : a.k;
  const uint16_t* in = isv ? a.vin : a.kin;
  AppendOneLoads L;
  L.vbyte[0] = L.vbyte[1] = 0;
  if (wave == 0 && !P.is_bf16 && P.tiled) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int bit;
      L.vbyte[i] = P.codes[vcode_byte(bh, a.cap, t, lane + 64 * i, D, &bit)];
    }
  }
  L.rr = load_r_rows<D, 4>(isv ? a.rv : a.rk);
  L.x = 0.0f;
  if (tid < D) L.x = bf16_to_f32(in[(((size_t)b * a.n_new + (t - T_old)) * a.Hkv + h) * D + tid]);
  return L;
}

template <bool CW>
__device__ __forceinline__ void append_one_finish(const AppendArgs& a, int bh, bool isv, int t, int T_old, int T_new,
                                         const AppendOneLoads& L, float* xs, float* part) {
  if (threadIdx.x < 128) xs[threadIdx.x] = L.x;
  __syncthreads();
  rotate_rows_regs<128, 4, 1>(xs, L.rr, part);
  __syncthreads();
  if ((threadIdx.x >> 6) != 0) return;
  append_tail<128, 4, 1, false, CW>(a, bh, isv, t, 1, T_old, T_new, part, L.vbyte);
}

// acc[j][c] += xs[j * xstride + e] * R[e][col + c] for e in [e0, e0 + EW)
// ascending (fused multiply-adds), c = 0, 1: one lane's share of a wave's
// part of a rotation whose reduction over e is split across waves.  The two
// columns are one 8-byte load per row; rows are loaded 32 at a time (one
// memory round trip per 32 rows).
template <int NX, int D, int EW = 128>
__device__ inline void rot_rows_cols2(const float* xs, int xstride, const float* R, int e0, int col,
                                      float (&acc)[NX][2]) {
  static_assert(EW % 32 == 0, "rows in batches of 32");
  const float* Rp = R + (size_t)e0 * D + col;
#pragma unroll 1
  for (int eb = 0; eb < EW; eb += 32) {
    float2 r[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) r[e] = *reinterpret_cast<const float2*>(Rp + (size_t)(eb + e) * D);
#pragma unroll
    for (int e = 0; e < 32; ++e)
#pragma unroll
      for (int j = 0; j < NX; ++j) {
        const float x = xs[j * xstride + e0 + eb + e];
        acc[j][0] = __builtin_fmaf(x, r[e].x, acc[j][0]);
        acc[j][1] = __builtin_fmaf(x, r[e].y, acc[j][1]);
      }
  }
}

// N rows of R (e0 .. e0 + N - 1, row length D) at columns col and col + 1,
// one 8-byte load per row, all issued together: a wave's share of a product
// whose reduction over e is split N rows per wave.
template <int N>
struct RowsN {
  float2 r[N];
};

template <int N>
__device__ inline RowsN<N> load_rows(const float* R, int D, int e0, int col) {
  RowsN<N> rr;
  const float* Rp = R + (size_t)e0 * D + col;
#pragma unroll
  for (int e = 0; e < N; ++e) rr.r[e] = *reinterpret_cast<const float2*>(Rp + (size_t)e * D);
  return rr;
}

// acc[j][c] += xs[j * xstride + e0 + e] * rows.r[e] (column c), e ascending
// (fused multiply-adds)
template <int NX, int N>
__device__ inline void fma_rows(const float* xs, int xstride, int e0, const RowsN<N>& rr, float (&acc)[NX][2]) {
#pragma unroll
  for (int e = 0; e < N; ++e)
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const float x = xs[j * xstride + e0 + e];
      acc[j][0] = __builtin_fmaf(x, rr.r[e].x, acc[j][0]);
      acc[j][1] = __builtin_fmaf(x, rr.r[e].y, acc[j][1]);
    }
}

// One-token append, head_dim 512, split by quantization group: the block
// computes dims [128 s, 128 s + 128) (group s) of one token row of plane K
// (isv = false) or V for one (sequence, kv head).  The rotation is the one of
// rotate_rows<512, 4, 1> for those dims (same waves, same order, same bits);
// the group's statistics, codes, scale|zero word and window values follow.
// Blocks of different groups touch disjoint bytes of every plane.  xs holds
// 512 floats and part 4 * 128 floats of shared memory.
template <bool LM = false>
__device__ inline void append_slice_block(const AppendArgs& a, int bh, bool isv, int s, float* xs, float* part) {
  constexpr int D = 512;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const PlaneDev P = isv ? a.v : a.k;
  const uint16_t* in = isv ? a.vin : a.kin;
  const float* R = isv ? a.rv : a.rk;
  float* dump = isv ? a.vdump : a.kdump;
  const int2 tr = append_range(a, b);
  const int t = tr.x;
  const size_t in_base = ((size_t)b * a.n_new * a.Hkv + h) * D;   // n_new == 1
  for (int i = tid; i < D; i += 256) xs[i] = bf16_to_f32(in[in_base + i]);
  __syncthreads();
  // lane computes columns 2 lane, 2 lane + 1 of the group's 128
  float acc[1][2] = {{0.0f, 0.0f}};
  rot_rows_cols2<1, D>(xs, 0, R, wave * 128, 128 * s + 2 * lane, acc);
  part[wave * 128 + 2 * lane] = acc[0][0];
  part[wave * 128 + 2 * lane + 1] = acc[0][1];
  __syncthreads();
  if (wave != 0) return;
  float x[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = lane + 64 * i;
    x[i] = (((part[d] + part[128 + d]) + part[256 + d]) + part[384 + d]) + 0.0f;
  }
  const int d0 = 128 * s + lane;      // dims d0 and d0 + 64 of the row
  if (dump) {
    const size_t base = ((size_t)b * a.n_new * a.Hkv + h) * D;
    dump[base + d0] = x[0];
    dump[base + d0 + 64] = x[1];
  }
  if (P.is_bf16) {
    const size_t base = row_offset(bh, a.cap, t, D);
    P.full[base + d0] = f32_to_bf16(x[0]);
    P.full[base + d0 + 64] = f32_to_bf16(x[1]);
    return;
  }
  if (t < a.N) {
    const size_t base = row_offset(bh, a.N, t, D);
    P.sink[base + d0] = f32_to_bf16(x[0]);
    P.sink[base + d0 + 64] = f32_to_bf16(x[1]);
  }
  if (a.M > 0 && t >= a.N && t >= tr.y - a.M) {
    const size_t base = row_offset(bh, a.M, t % a.M, D);
    P.ring[base + d0] = f32_to_bf16(x[0]);
    P.ring[base + d0 + 64] = f32_to_bf16(x[1]);
  }
  GroupQ q;
  uint32_t code[2];
  if constexpr (LM) {
    q = lm_group_wave(x[0], x[1], P.clip);
    code[0] = lm_code(x[0], q);
    code[1] = lm_code(x[1], q);
  } else {
    const float mx = wave_max(fmaxf(x[0], x[1]));
    const float mn = wave_min(fminf(x[0], x[1]));
    q = group_params(mx, mn, P.clip);
    code[0] = quant_code(x[0], q);
    code[1] = quant_code(x[1], q);
  }
  if (lane == 0) {
    P.meta[meta_index(bh, a.cap, t, s, D)] = q.packed;
    if (P.smax) atomicMax(reinterpret_cast<unsigned int*>(P.smax + bh), __float_as_uint(q.sf));
  }
  if (!P.tiled) {
    store_canonical<2>(code, lane, [&](int w) {
      return reinterpret_cast<uint32_t*>(P.codes + kcode_byte(bh, a.cap, t, 32 * s + 4 * w, D));
    });
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int bit;
      const size_t off = vcode_byte(bh, a.cap, t, d0 + 64 * i, D, &bit);
      const uint8_t old = P.codes[off];
      P.codes[off] = (uint8_t)((old & ~(3u << bit)) | (code[i] << bit));
    }
  }
}

}  // namespace oscar
