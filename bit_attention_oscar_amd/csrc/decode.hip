// Decode attention over the mixed INT2 + bf16 cache (split-K flash-decoding).
//
// Method (web pages on OSCAR): attention reads the 2-bit cache directly
// through a fused mixed-precision flash-attention ("OSCAR-LLAMACPP-Qwen3-4B-
// Thinking-2507-INT2-KV", "Run" env-var table; "OSCAR: 2-bit KV Cache
// Quantization for SGLang and llama.cpp", "How the offline rotation is fit");
// the first/last tokens are read from bf16 windows (Qwen3-4B card, "Run"
// table); q is rotated by R_K so q k^T is unchanged ("OSCAR-LLAMACPP-Gemma-4-
// 12B-it-INT2-KV", rotation paragraph below "Folders"); the V rotation is
// undone on the output ("OSCAR-RotationZoo", "How to use" step 2, the flag
// that absorbs it into the output projection).
//
// Kernels:
//   qrot_kernel         q_rot = q @ R_K * scale * log2(e) (fp32) for the general kernel
//   decode_valu_kernel  general split-K kernel: any head_dim / GQA / dtype /
//                       codebook (the only one for the Lloyd-Max codebook),
//                       per-token precision chosen by position
//   decode_prologue_kernel, decode_mfma_kernel
//                       head_dim 128, 4 or 8 query heads per kv head, INT2 K and
//                       V: INT2 splits with 16x16x32 f16 matrix-core QK^T and
//                       PV on the raw codes and two-piece q and softmax
//                       weights, bf16 window blocks, the merge and V
//                       un-rotation by the last block; q and a decode step's
//                       append either from the prologue launch or inside the
//                       attention launch (every block rotating its own q)
//   wide_qrot_kernel, wide_prologue_kernel, decode_wide_kernel
//                       head_dim 512 (q records, INT2 K with INT2 or bf16 V)
//   combine_kernel, combine_wide_kernel
//                       log-sum-exp merge of the splits and o = o' @ R_V^T
#include <math.h>
#include <algorithm>
#include <type_traits>
#include "append_impl.h"

namespace oscar {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

#define NEG_INF (-__builtin_inff())

// Scheduling fence between the phases of a tile (QK^T / softmax / PV): keeps
// the compiler from hoisting a whole tile of code conversions ahead of the
// softmax, which raises register pressure.
#define PHASE_FENCE() __builtin_amdgcn_sched_barrier(0)
// Waves per SIMD of the head_dim-128 attention kernel (its INT2 splits need
// about 160 registers: the PV accumulators, the tiles in flight, the softmax
// state).
constexpr int kMfmaWavesPerEu = 3;
// Register sets of tile data per wave: the loads of a tile are issued
// kDepth - 1 tiles ahead of its processing (head_dim 512 kernels).
constexpr int kDepth = 2;
// The same for the head_dim-128 INT2 splits: three sets (two tiles in flight
// while one is processed) measured 69.6 against 70.8 us per launch at the 32k
// shape; four sets at 2 waves per SIMD 69.0, five or more no faster.
constexpr int kDepth16 = 3;

__device__ inline float wmax(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// q rotation
// ---------------------------------------------------------------------------

// Matrix-core operand order.  QK^T runs 32 instructions per 64-token tile; the
// instruction for code word w (dims 16w..16w+15) and lane group pp takes the
// four k-slots
//   k0: d = 16w + 2pp      k1: d = 16w + 8 + 2pp
//   k2: d = 16w + 2pp + 1  k3: d = 16w + 9 + 2pp
// and the code operand of dim d carries a factor 4^(d % 4) (its bit position
// inside an fp16 denormal), so the q operand carries 4^-(d % 4).
__host__ __device__ inline int qk_dim(int w, int pp, int k) {
  return 16 * w + 2 * pp + (k & 2 ? 1 : 0) + (k & 1 ? 8 : 0);
}

// q rotation for the general kernel: one block per (sequence, kv head), its
// query heads in chunks of four, with the rotation routine of the append path
// (reduction over e split across the four waves, fixed-order partial sums).
template <int D>
__global__ __launch_bounds__(256) void qrot_kernel(QRotArgs a) {
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;        // b * Hkv + kvh
  const int b = bh / a.Hkv, kvh = bh - (bh / a.Hkv) * a.Hkv;
  const int Gq = a.Hq / a.Hkv;
  __shared__ float xs[4 * D];
  __shared__ float part[4 * 4 * D];
  for (int hc = 0; hc < Gq; hc += 4) {
    const int nh = min(4, Gq - hc);
    const int head0 = kvh * Gq + hc;
    for (int i = tid; i < 4 * D; i += 256) {
      const int j = i / D, d = i - (i / D) * D;
      xs[i] = j < nh ? bf16_to_f32(a.q[((size_t)b * a.Hq + head0 + j) * D + d]) : 0.0f;
    }
    __syncthreads();
    rotate_rows<D, 4, 4>(xs, a.rk, part, 4);
    __syncthreads();
    for (int i = tid; i < nh * D; i += 256) {
      const int j = i / D, d = i - (i / D) * D;
      a.qrot[((size_t)b * a.Hq + head0 + j) * D + d] = rot_sum<D, 4, 4>(part, j, d) * a.scale_log2;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// general VALU split-K kernel
// ---------------------------------------------------------------------------

// value of code c in units of the group's step: c (min/max codebook) or the
// Lloyd-Max level
__device__ inline float code_value(const PlaneDev& P, uint32_t c) {
  return P.lm ? lm_level(c) : (float)c;
}

template <int D>
__device__ inline void load_row_values(const PlaneDev& P, int bh, int t, int T, int N, int M, int cap,
                                       int d0, int n, float* out) {
  // n consecutive dims starting at d0 (n multiple of 8, within one group)
  const bool hp = P.is_bf16 || t < N || t >= T - M;
  if (hp) {
    const uint16_t* row = P.is_bf16 ? P.full + row_offset(bh, cap, t, D)
                          : (t < N ? P.sink + row_offset(bh, N, t, D) : P.ring + row_offset(bh, M, t % M, D));
    for (int i = 0; i < n; i += 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + d0 + i);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[i + 2 * k] = bf16_to_f32((uint16_t)(w[k] & 0xFFFFu));
        out[i + 2 * k + 1] = bf16_to_f32((uint16_t)(w[k] >> 16));
      }
    }
    return;
  }
  const uint32_t meta = P.meta[meta_index(bh, cap, t, d0 / kGroup, D)];
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta >> 16));
  if (!P.tiled) {
    for (int i = 0; i < n; i += 16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(P.codes + kcode_byte(bh, cap, t, (d0 + i) / 4, D));
#pragma unroll
      for (int k = 0; k < 16; ++k) out[i + k] = __builtin_fmaf(s, code_value(P, (w >> (2 * k)) & 3u), z);
    }
  } else {
    for (int i = 0; i < n; ++i) {
      int bit;
      const size_t off = vcode_byte(bh, cap, t, d0 + i, D, &bit);
      out[i] = __builtin_fmaf(s, code_value(P, (P.codes[off] >> bit) & 3u), z);
    }
  }
}

template <int D>
__device__ inline float load_value(const PlaneDev& P, int bh, int t, int T, int N, int M, int cap, int d) {
  const bool hp = P.is_bf16 || t < N || t >= T - M;
  if (hp) {
    const uint16_t* row = P.is_bf16 ? P.full + row_offset(bh, cap, t, D)
                          : (t < N ? P.sink + row_offset(bh, N, t, D) : P.ring + row_offset(bh, M, t % M, D));
    return bf16_to_f32(row[d]);
  }
  const uint32_t meta = P.meta[meta_index(bh, cap, t, d / kGroup, D)];
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta >> 16));
  uint32_t c;
  if (!P.tiled) {
    c = (P.codes[kcode_byte(bh, cap, t, d / 4, D)] >> (2 * (d & 3))) & 3u;
  } else {
    int bit;
    const size_t off = vcode_byte(bh, cap, t, d, D, &bit);
    c = (P.codes[off] >> bit) & 3u;
  }
  return __builtin_fmaf(s, code_value(P, c), z);
}

__device__ inline int seg_token(const SegPlan& p, int vt) {
  const int len0 = p.b0 - p.a0;
  return vt < len0 ? p.a0 + vt : p.a1 + (vt - len0);
}

template <int D>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  constexpr int DC = (D + 255) / 256;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const int Gq = a.Hq / a.Hkv;
  const int split = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ float qs[kMaxGq][D];
  __shared__ float ps[kMaxGq][64];
  __shared__ float ms[kMaxGq], ls[kMaxGq], al[kMaxGq];

  for (int i = tid; i < Gq * D; i += 256) {
    const int hq = i / D, d = i - hq * D;
    qs[hq][d] = a.qrot[((size_t)b * a.Hq + h * Gq + hq) * D + d];
  }
  if (tid < kMaxGq) {
    ms[tid] = NEG_INF;
    ls[tid] = 0.0f;
  }
  float o[kMaxGq][DC];
#pragma unroll
  for (int hq = 0; hq < kMaxGq; ++hq)
#pragma unroll
    for (int c = 0; c < DC; ++c) o[hq][c] = 0.0f;
  __syncthreads();

  // tokens of this sequence (ragged batch: its own count; the plan then
  // covers the longest sequence, [0, T) in one segment)
  const int T = a.lens ? a.lens[b] : a.T;
  const int len = a.lens ? T : (a.plan.b0 - a.plan.a0) + (a.plan.b1 - a.plan.a1);
  const int v_lo = split * a.plan.chunk;
  const int v_hi = min(v_lo + a.plan.chunk, len);
  constexpr int PART = D / 4;  // dims per thread in the score phase
  for (int vt0 = v_lo; vt0 < v_hi; vt0 += 64) {
    // scores: thread (token tok, quarter part) over dims [part*D/4, (part+1)*D/4)
    {
      const int tok = tid >> 2, part = tid & 3;
      const int vt = vt0 + tok;
      float dots[kMaxGq];
#pragma unroll
      for (int hq = 0; hq < kMaxGq; ++hq) dots[hq] = 0.0f;
      if (vt < v_hi) {
        const int t = seg_token(a.plan, vt);
        for (int c0 = 0; c0 < PART; c0 += 16) {
          float kv[16];
          load_row_values<D>(a.k, bh, t, T, a.N, a.M, a.cap, part * PART + c0, 16, kv);
#pragma unroll
          for (int hq = 0; hq < kMaxGq; ++hq) {
            if (hq < Gq) {
              float s = dots[hq];
#pragma unroll
              for (int k = 0; k < 16; ++k) s = __builtin_fmaf(qs[hq][part * PART + c0 + k], kv[k], s);
              dots[hq] = s;
            }
          }
        }
      }
#pragma unroll
      for (int hq = 0; hq < kMaxGq; ++hq) {
        dots[hq] += __shfl_xor(dots[hq], 1);
        dots[hq] += __shfl_xor(dots[hq], 2);
      }
      if (part == 0) {
        for (int hq = 0; hq < Gq; ++hq) ps[hq][tok] = (vt < v_hi) ? dots[hq] : NEG_INF;
      }
    }
    __syncthreads();
    // online softmax update per head (log2 domain)
    for (int hq = wave; hq < Gq; hq += 4) {
      const float s = ps[hq][lane];
      const float mx = wmax(s);
      const float mold = ms[hq];
      const float mnew = fmaxf(mold, mx);
      const float p = (s == NEG_INF) ? 0.0f : exp2f(s - mnew);
      const float sum = wsum(p);
      ps[hq][lane] = p;
      if (lane == 0) {
        const float alpha = (mold == NEG_INF) ? 0.0f : exp2f(mold - mnew);
        al[hq] = alpha;
        ms[hq] = mnew;
        ls[hq] = ls[hq] * alpha + sum;
      }
    }
    __syncthreads();
    // PV: thread owns dims tid + 256 c
#pragma unroll
    for (int hq = 0; hq < kMaxGq; ++hq)
      if (hq < Gq)
#pragma unroll
        for (int c = 0; c < DC; ++c) o[hq][c] *= al[hq];
    const int ntk = min(64, v_hi - vt0);
    for (int tk = 0; tk < ntk; ++tk) {
      const int t = seg_token(a.plan, vt0 + tk);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const int d = tid + 256 * c;
        if (d < D) {
          const float vv = load_value<D>(a.v, bh, t, T, a.N, a.M, a.cap, d);
#pragma unroll
          for (int hq = 0; hq < kMaxGq; ++hq)
            if (hq < Gq) o[hq][c] = __builtin_fmaf(ps[hq][tk], vv, o[hq][c]);
        }
      }
    }
    __syncthreads();
  }
  const int slot = a.plan.slot0 + split;
  for (int hq = 0; hq < Gq; ++hq) {
    float* dst = a.partials + (((size_t)b * a.Hq + h * Gq + hq) * a.pstride + slot) * (D + 2);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int d = tid + 256 * c;
      if (d < D) dst[d] = o[hq][c];
    }
    if (tid == 0) {
      dst[D] = ms[hq];
      dst[D + 1] = ls[hq];
    }
  }
}

// ---------------------------------------------------------------------------
// matrix-core INT2 kernel (head_dim 128, 4 query heads per kv head)
// ---------------------------------------------------------------------------
//
// Wave = 64 lanes = 16 blocks of the 4x4x4 instruction; lane = 4*blk + col.
// QK^T: A = codes of token (tile + lane) (row = token in block, k = 4 dims),
//       B = q operand (col = query head), broadcast from lane group pp;
//       32 instructions cover 128 dims; output lane (blk, j) register r =
//       score of token tile + 4 blk + r for head j.
// PV:   A = p * s_V (row = head, k = 4 tokens of block beta), broadcast from
//       block beta; B = V codes (col = dim); 16 betas x 2 halves of head_dim;
//       output lane (blk, jj) register r = o'[head r][64 hh + 4 blk + jj].
// A code c enters an instruction as the fp16 denormal c * 4^s * 2^-24 (one AND
// of the packed word; s = bit pair inside the byte); the other operand carries
// 4^-s and a power of two that keeps it in the fp16 normal range.

__device__ inline h4 as_h4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(h4, (uint64_t)lo | ((uint64_t)hi << 32));
}

__device__ inline void split_codes(uint32_t w, uint32_t c[8]) {
  const uint32_t u = w >> 8;
  c[0] = w & 0x00030003u;
  c[1] = w & 0x000C000Cu;
  c[2] = w & 0x00300030u;
  c[3] = w & 0x00C000C0u;
  c[4] = u & 0x00030003u;
  c[5] = u & 0x000C000Cu;
  c[6] = u & 0x00300030u;
  c[7] = u & 0x00C000C0u;
}

__device__ inline float lo_half(uint32_t m) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFFu)); }
__device__ inline float hi_half(uint32_t m) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(m >> 16)); }

// Two-piece fp16 operands.  A value x that enters a product as fp16 is
// carried as hi = fp16(x) and lo = fp16(x - hi) (x - hi is exact in fp32), so
// the operand keeps 22 significant bits instead of 11; both pieces multiply
// the same exact code operand and accumulate into the same fp32 chain.  With
// one fp16 piece the scores of large-magnitude q (outlier channels) carry an
// absolute error proportional to their size, which the softmax exponentiates.
__device__ inline void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// Word w of a lane's K codes against the q operands of every head group: the
// codes are unpacked once, each group has its own accumulation chain, which
// takes the high pieces (registers) and then the low pieces (read from the
// block's shared copy, qlo[g] = this lane's 8 words of group g).
template <int G>
__device__ inline void qk_word(uint32_t word, const h4 (&q)[G][8], const uint2* const (&qlo)[G], int w,
                               f4 (&s)[G]) {
  uint32_t c[8];
  split_codes(word, c);
  h4 ql[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint2 u = qlo[g][w];
    ql[g] = as_h4(u.x, u.y);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[0], c[1]), q[g][w], s[g], 0, 0, 4);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[2], c[3]), q[g][w], s[g], 0, 0, 5);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[4], c[5]), q[g][w], s[g], 0, 0, 6);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[6], c[7]), q[g][w], s[g], 0, 0, 7);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[0], c[1]), ql[g], s[g], 0, 0, 4);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[2], c[3]), ql[g], s[g], 0, 0, 5);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[4], c[5]), ql[g], s[g], 0, 0, 6);
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[6], c[7]), ql[g], s[g], 0, 0, 7);
}

// PV for word W of a lane's V record with the two-piece weights p (high) and
// pl (low) of every head group.
template <int G, int W>
__device__ inline void pv_word(uint32_t word, const h4 (&p)[G], const h4 (&pl)[G], f4 (&o0)[G], f4 (&o1)[G]) {
  uint32_t c[8];
  split_codes(word, c);
  // word W holds tokens 8W..8W+7 = blocks beta 2W (pairs 0,1) and 2W+1 (pairs 2,3);
  // positions 0-3 are the low half of head_dim, 4-7 the high half
#pragma unroll
  for (int g = 0; g < G; ++g) {
    o0[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(p[g], as_h4(c[0], c[1]), o0[g], 4, 2 * W, 0);
    o1[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(p[g], as_h4(c[4], c[5]), o1[g], 4, 2 * W, 0);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    o0[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(p[g], as_h4(c[2], c[3]), o0[g], 4, 2 * W + 1, 0);
    o1[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(p[g], as_h4(c[6], c[7]), o1[g], 4, 2 * W + 1, 0);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    o0[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(pl[g], as_h4(c[0], c[1]), o0[g], 4, 2 * W, 0);
    o1[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(pl[g], as_h4(c[4], c[5]), o1[g], 4, 2 * W, 0);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    o0[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(pl[g], as_h4(c[2], c[3]), o0[g], 4, 2 * W + 1, 0);
    o1[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(pl[g], as_h4(c[6], c[7]), o1[g], 4, 2 * W + 1, 0);
  }
}

// The softmax weights of four tokens as two-piece PV operands: s_V * p' with
// one fp32 rounding (the fp16 scale read in place), split into hi and lo.
__device__ inline void pv_operands(const uint32_t (&vmr)[4], const float (&p)[4], h4& hi, h4& lo) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    _Float16 h, l;
    split_f16(__builtin_fmaf(lo_half(vmr[r]), p[r], 0.0f), h, l);
    hi[r] = h;
    lo[r] = l;
  }
}

// ---------------------------------------------------------------------------
// combine + V un-rotation
// ---------------------------------------------------------------------------

// One block per (sequence, kv head): merge the splits of its query heads
// (chunks of four), then o = o' @ R_V^T with the reduction over e split across
// the four waves.
// Partial loads: plain, or device-scope (coherent across XCDs within a launch).
template <bool COHERENT>
__device__ inline float ld_partial(const float* p) {
  if (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
// two consecutive partial floats (8-byte aligned) in one device-scope load
__device__ inline float2 ld_partial2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// One output element in the requested dtype.
__device__ inline void store_out(const CombineArgs& a, size_t o, float v) {
  if (a.out_dtype == 0)
    reinterpret_cast<float*>(a.out)[o] = v;
  else if (a.out_dtype == 1)
    reinterpret_cast<uint16_t*>(a.out)[o] = f32_to_bf16(v);
  else
    reinterpret_cast<uint16_t*>(a.out)[o] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// CC > 1: the block computes output columns [cc D / CC, (cc + 1) D / CC) only
// (it still merges every dim of o', which the un-rotation reduces over).
// Query heads [h_begin, h_end) of the kv head (all of them by default).
template <int D, bool COHERENT = false, int CC = 1>
__device__ void combine_group(const CombineArgs& a, int bh, int cc = 0, int h_begin = 0, int h_end = -1) {
  constexpr int NC = D / CC;          // output columns of the block
  constexpr int PER = NC / 64;
  constexpr int EW = D / 4;
  static_assert(NC % 64 == 0, "column chunk");
  const int c0 = cc * NC;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = bh / a.Hkv, kvh = bh - (bh / a.Hkv) * a.Hkv;
  const int Gq = a.Hq / a.Hkv;
  __shared__ float wsl[4][kMaxSplits];
  __shared__ float linv[4];
  __shared__ float os[4][D];
  __shared__ float part[4][4][NC];
  if (h_end < 0) h_end = Gq;
  for (int hc = h_begin; hc < h_end; hc += 4) {
    const int nh = min(4, h_end - hc);
    // split weights: wave j handles head j; every (m, l) pair of a lane is
    // loaded in one round trip (at most kMaxSplits / 64 slots per lane)
    if (wave < nh) {
      const float* P = a.partials + ((size_t)b * a.Hq + kvh * Gq + hc + wave) * a.pstride * (D + 2);
      constexpr int SPL = kMaxSplits / 64;
      float ms[SPL], ls[SPL];
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int sl = lane + 64 * i;
        ms[i] = NEG_INF;
        ls[i] = 0.0f;
        if (sl < a.nslots) {
          ms[i] = ld_partial<COHERENT>(P + (size_t)sl * (D + 2) + D);
          ls[i] = ld_partial<COHERENT>(P + (size_t)sl * (D + 2) + D + 1);
        }
      }
      float mx = NEG_INF;
#pragma unroll
      for (int i = 0; i < SPL; ++i) mx = fmaxf(mx, ms[i]);
      const float M = wmax(mx);
      float L = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int sl = lane + 64 * i;
        const float w = (ms[i] == NEG_INF) ? 0.0f : exp2f(ms[i] - M);
        if (sl < a.nslots) wsl[wave][sl] = w;
        L = __builtin_fmaf(ls[i], w, L);
      }
      L = wsum(L);
      if (lane == 0) linv[wave] = 1.0f / L;
    }
    __syncthreads();
    // merged o': thread (j, d pair); 32 slots' loads in flight per step; past
    // the last slot the index is clamped (a valid address) and the weight is zero
    for (int idx = tid; idx < 2 * D; idx += 256) {
      const int j = idx / (D / 2), d = 2 * (idx - j * (D / 2));
      float acc0 = 0.0f, acc1 = 0.0f;
      if (j < nh) {
        const float* P = a.partials + ((size_t)b * a.Hq + kvh * Gq + hc + j) * a.pstride * (D + 2);
        for (int sl = 0; sl < a.nslots; sl += 32) {
          float v[32][2];
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            const float* src = P + (size_t)min(sl + u, a.nslots - 1) * (D + 2) + d;
            v[u][0] = ld_partial<COHERENT>(src);
            v[u][1] = ld_partial<COHERENT>(src + 1);
          }
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            const float w = sl + u < a.nslots ? wsl[j][min(sl + u, a.nslots - 1)] : 0.0f;
            acc0 = __builtin_fmaf(v[u][0], w, acc0);
            acc1 = __builtin_fmaf(v[u][1], w, acc1);
          }
        }
        acc0 *= linv[j];
        acc1 *= linv[j];
      }
      os[j][d] = acc0;
      os[j][d + 1] = acc1;
    }
    __syncthreads();
    if (a.absorb_v) {                     // o' in the V-rotated basis, this block's columns
      for (int idx = tid; idx < nh * NC; idx += 256) {
        const int j = idx / NC, d = idx - (idx / NC) * NC;
        store_out(a, ((size_t)b * a.Hq + kvh * Gq + hc + j) * D + c0 + d, os[j][c0 + d]);
      }
      __syncthreads();
      continue;
    }
    // o = o' @ R_V^T for this block's columns: lane pair-columns 2 lane + 128 i
#pragma unroll
    for (int i = 0; i < PER / 2; ++i) {
      float acc[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j][0] = acc[j][1] = 0.0f;
      rot_rows_cols2<4, D, EW>(&os[0][0], D, a.rvT, wave * EW, c0 + 128 * i + 2 * lane, acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part[wave][j][128 * i + 2 * lane] = acc[j][0];
        part[wave][j][128 * i + 2 * lane + 1] = acc[j][1];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < nh * NC; idx += 256) {
      const int j = idx / NC, d = idx - (idx / NC) * NC;
      const float v = ((part[0][j][d] + part[1][j][d]) + part[2][j][d]) + part[3][j][d];
      store_out(a, ((size_t)b * a.Hq + kvh * Gq + hc + j) * D + c0 + d, v);
    }
    __syncthreads();
  }
}

// Grid: (sequence x kv head, CC column chunks of the output, query-head
// blocks of HB heads).  At head_dim 512 one head per block: a merge is a few
// dependent memory round trips long, and more, smaller blocks fill more of the
// compute units.
template <int D, int CC, int HB>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int h0 = (int)blockIdx.z * HB;
  combine_group<D, false, CC>(a, (int)blockIdx.x, (int)blockIdx.y, h0, min(h0 + HB, a.Hq / a.Hkv));
}

// Merge and V un-rotation at head_dim 512: block (sequence x kv head, column
// chunk cc of 128, query head j of the kv head), 8 waves, one memory round
// trip for every load: wave w's R_Vᵀ rows [64 w, 64 w + 64) at the block's
// columns 2 lane, 2 lane + 1; wave 0's (m, l) of every slot (lane s: slots s,
// s + 64, ...); and o': thread t (t % 256 = dim pair p, t / 256 = slot group
// g) loads dims 2p, 2p + 1 of slots [32 g, 32 g + 32) of each round of 64
// slots.  The weighted sums of the two slot groups are added in group order,
// the 8 waves' partial products in wave order.
__global__ __launch_bounds__(512) void combine_wide_kernel(CombineArgs a) {
  constexpr int D = 512, NC = 128, WAVES = 8, RW = D / WAVES, SG = 512 / 256, SU = 64 / SG;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = (int)blockIdx.x, c0 = (int)blockIdx.y * NC, j = (int)blockIdx.z;
  const int b = bh / a.Hkv, kvh = bh - (bh / a.Hkv) * a.Hkv;
  const int Gq = a.Hq / a.Hkv, hq = kvh * Gq + j, ns = a.nslots;
  const float* P = a.partials + ((size_t)b * a.Hq + hq) * a.pstride * (D + 2);
  __shared__ float wsl[kMaxSplits + 64];  // m, then the slot weight
  __shared__ float wll[kMaxSplits + 64];  // l
  __shared__ float linv;
  __shared__ float os[SG][D];
  __shared__ float part[WAVES][NC];
  const RowsN<RW> rr = load_rows<RW>(a.rvT, D, RW * wave, c0 + 2 * lane);
  const int pr = tid & 255, grp = tid >> 8;
  float o0 = 0.0f, o1 = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float2 v[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u)
      v[u] = ld_partial2(P + (size_t)min(s0 + SU * grp + u, ns - 1) * (D + 2) + 2 * pr);
    if (s0 == 0) {
      if (wave == 0) {
        // slot weights relative to the maximum m, and 1 / l (lane s: slots
        // s, s + 64, ...; one round of loads up to 64 slots)
        float mx = NEG_INF;
        for (int i = 0; 64 * i < ns; ++i) {
          const int sl = lane + 64 * i;
          const float2 t = ld_partial2(P + (size_t)min(sl, ns - 1) * (D + 2) + D);
          wsl[sl] = t.x;
          wll[sl] = t.y;
          if (sl < ns) mx = fmaxf(mx, t.x);
        }
        const float M = wmax(mx);
        float L = 0.0f;
        for (int i = 0; 64 * i < ns; ++i) {
          const int sl = lane + 64 * i;
          const float m = wsl[sl];
          const float w = (sl >= ns || m == NEG_INF) ? 0.0f : exp2f(m - M);
          wsl[sl] = w;
          L = __builtin_fmaf(wll[sl], w, L);
        }
        L = wsum(L);
        if (lane == 0) linv = 1.0f / L;
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int sl = s0 + SU * grp + u;
      const float w = sl < ns ? wsl[sl] : 0.0f;
      o0 = __builtin_fmaf(v[u].x, w, o0);
      o1 = __builtin_fmaf(v[u].y, w, o1);
    }
  }
  os[grp][2 * pr] = o0;
  os[grp][2 * pr + 1] = o1;
  __syncthreads();
  if (tid < D) os[0][tid] = (os[0][tid] + os[1][tid]) * linv;
  __syncthreads();
  const size_t orow = ((size_t)b * a.Hq + hq) * D;
  if (a.absorb_v) {                       // o' in the V-rotated basis, this block's columns
    if (tid < NC) store_out(a, orow + c0 + tid, os[0][c0 + tid]);
    return;
  }
  float acc[1][2] = {{0.0f, 0.0f}};
  fma_rows<1, RW>(&os[0][0], 0, RW * wave, rr, acc);
  part[wave][2 * lane] = acc[0][0];
  part[wave][2 * lane + 1] = acc[0][1];
  __syncthreads();
  if (tid < NC) {
    float v = part[0][tid];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v = v + part[w][tid];
    store_out(a, orow + c0 + tid, v);
  }
}

// Partial results of the matrix-core launch are written with device-scope
// stores, which complete at the level shared by all XCDs.
__device__ inline void st_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every block of the matrix-core launch after it wrote its partial:
// the last block to finish for a (sequence, kv head) merges all of them.
// Every thread waits for its device-scope partial stores to complete before the
// barrier, then one thread increments the counter; the last block reads the
// partials with device-scope loads.  No cache-wide write-back or invalidation,
// and no block ever waits for another.
struct FusedSmem;
template <int D, int WAVES>
struct RRows;
template <int G>
__device__ void combine_fused(const CombineArgs& a, int bh, FusedSmem& S);
__device__ __forceinline__ void combine_group4(const CombineArgs& a, int b, int hq0, FusedSmem& S);

template <int G>
__device__ inline void finish_block(const DecodeArgs& a, int bh, FusedSmem& S) {
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned total = (unsigned)(a.one_round ? a.plan.splits : a.plan.splits + a.win_blocks);
    const unsigned prev = __hip_atomic_fetch_add(a.counters + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == total - 1u);
  }
  __syncthreads();
  if (!is_last) return;
  combine_fused<G>(a.comb, bh, S);
  if (threadIdx.x == 0) {
    if (a.app_blocks > 0) {
      // the appended token's V scale joins the running maximum only now, when
      // no block of the launch reads the maximum any more (the block that
      // appended counted itself after its stores completed)
      unsigned* pend = reinterpret_cast<unsigned*>(a.app.v.smax + bh);
      const unsigned sf = __hip_atomic_load(pend, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_max(reinterpret_cast<unsigned*>(a.v.smax + bh), sf, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pend, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// bf16 window tokens (sink + recent) of one (sequence, kv head): one block of
// 256 threads takes up to 64 of them with fp32 VALU arithmetic.  Every row load
// of a phase is issued before its arithmetic.
__device__ inline int win_token(const SegPlan& w, int vt) {
  const int len0 = w.b0 - w.a0;
  return vt < len0 ? w.a0 + vt : w.a1 + (vt - len0);
}

// The token sets of the block's sequence: its length, the end of its INT2
// range [plan.a0, hi), its window segments [0, win.b0) and [win.a1, T) (with
// the launch's chunk, splits and first slot) and the ring slot of win.a1.  In
// a ragged batch every sequence has its own; the host's plan is that of the
// longest, which sizes the grid, and blocks past a shorter sequence's tokens
// find empty ranges.
struct SeqView {
  int T, hi, ring0;
  SegPlan win;
};

__device__ inline SeqView seq_view(const DecodeArgs& a, int b) {
  SeqView v;
  v.win = a.win;
  if (!a.lens) {
    v.T = a.T;
    v.hi = a.plan.b0;
    v.ring0 = a.ring0;
    return v;
  }
  const int T = a.lens[b];
  v.T = T;
  v.hi = max(a.N, T - a.M);
  v.win.a0 = 0;
  v.win.b0 = min(a.N, T);
  v.win.a1 = min(T, max(a.N, T - a.M));        // below N tokens: empty
  v.win.b1 = T;
  v.ring0 = a.M > 0 ? v.win.a1 % a.M : 0;
  return v;
}

// Row of window token t: sink row t, or ring slot t % M.  The recent tokens
// are consecutive from win.a1, whose slot is ring0, so no division is needed.
__device__ inline const uint16_t* win_row(const DecodeArgs& a, const SeqView& sv, const PlaneDev& P, int bh, int t) {
  constexpr int D = 128;
  if (t < a.N) return P.sink + row_offset(bh, a.N, t, D);
  int slot = sv.ring0 + (t - sv.win.a1);
  if (slot >= a.M) slot -= a.M;
  return P.ring + row_offset(bh, a.M, slot, D);
}

__device__ inline void bf16x8(const uint4 u, float* x);
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
__device__ inline void bf16x8(const u4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
}
__device__ inline void bf16x8(const uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
}

// Shared memory of the head_dim-128 launches; each block role uses its own regions and
// the scratch area is reused phase by phase.
struct FusedSmem {
  float qs[4][132];            // rotated q of the block's 4 heads (fp32, x scale*log2 e)
  float qsum[4];               // per-head sums of qs
  int qeq[4];                  // per-head exponent of the fp16 q operand
  uint32_t meta16[4][128];     // INT2 splits: per wave, the K and V scale|zero words of a tile
  u4 qops[8][64];              // INT2 splits: q operand n of lane l (the same in every wave)
  float scratch[2688];
};

// q rotation of the block's 4 query heads, in two steps so that a block can
// issue every load it needs at once (one memory round trip) and put other
// loads behind them before it waits: the raw q rows (two values per thread)
// and this lane's rows of R_K (its wave's quarter of e, dims lane and
// lane + 64).  The arithmetic is the append path's rotation routine's: fmas
// over e ascending per wave, the four partial sums added in a fixed order.
struct QRotLoads {
  float q0, q1;
  float r[32][2];
};

__device__ inline QRotLoads q_rotation_loads(const DecodeArgs& a, int b, int hq0) {
  constexpr int D = 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  QRotLoads s;
  const uint16_t* qb = a.q + ((size_t)b * a.Hq + hq0) * D;       // the group's 4 heads' rows, contiguous
  s.q0 = bf16_to_f32(qb[tid]);
  s.q1 = bf16_to_f32(qb[tid + 256]);
  const float* Rw = a.rk + (size_t)(wave * 32) * D + lane;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    s.r[e][0] = Rw[(size_t)e * D];
    s.r[e][1] = Rw[(size_t)e * D + 64];
  }
  return s;
}

__device__ __forceinline__ void q_rotation_finish(const DecodeArgs& a, const QRotLoads& s, FusedSmem& S) {
  constexpr int D = 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float* qraw = S.scratch;            // [4][128]
  float* part = S.scratch + 512;      // [4 waves][4][128]
  qraw[tid] = s.q0;
  qraw[tid + 256] = s.q1;
  __syncthreads();
  float acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j][0] = acc[j][1] = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = qraw[j * D + wave * 32 + e];
      acc[j][0] = __builtin_fmaf(x, s.r[e][0], acc[j][0]);
      acc[j][1] = __builtin_fmaf(x, s.r[e][1], acc[j][1]);
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    part[(wave * 4 + j) * D + lane] = acc[j][0];
    part[(wave * 4 + j) * D + lane + 64] = acc[j][1];
  }
  __syncthreads();
  {
    const int j = wave;                // wave j finishes head j
    const float v0 = rot_sum<128, 4, 4>(part, j, lane) * a.scale_log2;
    const float v1 = rot_sum<128, 4, 4>(part, j, lane + 64) * a.scale_log2;
    S.qs[j][lane] = v0;
    S.qs[j][lane + 64] = v1;
    const float sum = wsum(v0 + v1);
    const float amax = wmax(fmaxf(fabsf(v0), fabsf(v1)));
    int e2 = 0;
    if (amax > 0.0f) frexpf(amax, &e2);
    if (lane == 0) {
      S.qsum[j] = sum;
      S.qeq[j] = (amax > 0.0f) ? 15 - e2 : 0;     // |q| * 2^eq < 2^15
    }
  }
  __syncthreads();
}

// fp16 matrix-core q operand pieces: element k of word w for lane group pp of
// head j is x = q_rot[d] * 2^(eq - 2 (d % 4)) with d = qk_dim(w, pp, k), as
// hi = fp16(x) and lo = fp16(x - hi).
__device__ inline void q_operand(const FusedSmem& S, int j, int pp, int w, int k, _Float16& hi, _Float16& lo) {
  const int d = qk_dim(w, pp, k);
  split_f16(ldexpf(S.qs[j][d], S.qeq[j] - 2 * (d & 3)), hi, lo);
}

// Published q of one head group (4 query heads) of a (sequence, kv head), at
// index (b Hkv + h) G + g, kQPub floats:
//   [0, 512)          fp32 rotated q of the 4 heads, head-major
//   [512, 516)        per-head sums; [516, 520) per-head exponents eq (int bits)
//   [kQPubOps, +256)  head_dim 512 records: high pieces of the fp16 operands
//                     of the 4x4x4 products: vector 4 pp + j holds the 32
//                     values (word w, slot k at 4 w + k) of lane group pp,
//                     head j (16 words per vector)
//   [kQPubLo, +256)   the low pieces, same order
//   [kQPub16, +512)   head_dim 128 records: both pieces of the operands of the
//                     16x16x32 products (publish_q)
constexpr int kQPubOps = 520;
constexpr int kQPubLo = kQPubOps + 256;
constexpr int kQPub16 = kQPubLo + 256;
static_assert(kQPub16 + 512 <= kQPub, "published q layout");

// Word i (0 <= i < 256) of the operand vectors of the block's 4 heads, as
// published: vector v = i / 16 = 4 pp + j, operands 2 (i % 16) and
// 2 (i % 16) + 1 of that vector; hw packs the two high pieces, lw the two low.
__device__ inline void q_operand_word(const FusedSmem& S, int i, uint32_t& hw, uint32_t& lw) {
  const int v = i >> 4, e = 2 * (i & 15);
  const int pp = v >> 2, j = v & 3;
  _Float16 h0, l0, h1, l1;
  q_operand(S, j, pp, e >> 2, e & 3, h0, l0);
  q_operand(S, j, pp, (e + 1) >> 2, (e + 1) & 3, h1, l1);
  hw = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  lw = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// Two fp16 q operand items (2d, 2d + 1) of chunk kc for lane group g, head j,
// piece `piece`: dims 16 w + 4 hf + d and 16 w + 8 + 4 hf + d (w = 2 g +
// kc/2, hf = kc % 2), times 2^(eq - 2d), packed low | high.
__device__ inline uint32_t q_operand16_pair(const FusedSmem& S, int j, int g, int piece, int kc, int d) {
  const int w = 2 * g + (kc >> 1), hf = kc & 1;
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    _Float16 hi, lo;
    split_f16(ldexpf(S.qs[j][16 * w + 8 * e + 4 * hf + d], S.qeq[j] - 2 * d), hi, lo);
    out |= (uint32_t)__builtin_bit_cast(uint16_t, piece ? lo : hi) << (16 * e);
  }
  return out;
}

// The q record of one head group, written by the q-record launch for the
// attention launch: the fp32 part and the operand pieces of the instruction
// shape that launch uses (FOUR: the 4x4x4 products of the head_dim-512
// kernels; else the 16x16x32 products of the head_dim-128 kernel).
template <bool FOUR>
__device__ __forceinline__ void publish_q(const DecodeArgs& a, int pidx, FusedSmem& S) {
  float* dst = a.qpub + (size_t)pidx * kQPub;
  const int tid = threadIdx.x;
  for (int i = tid; i < 4 * 128; i += blockDim.x) st_partial(dst + i, S.qs[i >> 7][i & 127]);
  if (tid < 4) {
    st_partial(dst + 512 + tid, S.qsum[tid]);
    st_partial(dst + 516 + tid, __int_as_float(S.qeq[tid]));
  }
  if constexpr (FOUR) {
    if (tid < 256) {                    // one word (two fp16 operands) of each piece per thread
      uint32_t hw, lw;
      q_operand_word(S, tid, hw, lw);
      st_partial(dst + kQPubOps + tid, __uint_as_float(hw));
      st_partial(dst + kQPubLo + tid, __uint_as_float(lw));
    }
  } else {
    // operands of the 16x16x32 products: vector (piece 4 + g) 4 + j holds
    // word 4 kc + d = items (2d, 2d + 1) of chunk kc for lane group g, head j
    for (int i = tid; i < 512; i += blockDim.x) {
      const int v = i >> 4, wd = i & 15;
      st_partial(dst + kQPub16 + i,
                 __uint_as_float(q_operand16_pair(S, v & 3, (v >> 2) & 3, v >> 4, wd >> 2, wd & 3)));
    }
  }
}

// Merge of the (m, l, o') partials of one (sequence, kv head) by the last
// block of the matrix-core launch, then o = o' @ R_V^T (4 query heads per kv
// head, head_dim 128; combine_group4).  The rotation splits its reduction
// over e across the four waves and adds the partial sums in a fixed order.
template <int G>
__device__ void combine_fused(const CombineArgs& a, int bh, FusedSmem& S) {
  const int b = bh / a.Hkv, kvh = bh - (bh / a.Hkv) * a.Hkv;
#pragma unroll
  for (int g = 0; g < G; ++g) combine_group4(a, b, kvh * 4 * G + 4 * g, S);
}

// One-round-trip merge of up to SF slots for head `wave` (lane l: dims 2 l and
// 2 l + 1): lane s < ns loads slot s's m and l, every lane loads its two dims of
// every slot's o' (one 8-byte load each), all in flight together; the slot
// weights are formed in the lanes that hold them and read by every lane
// (v_readlane), and o' is summed in slot order.
template <int SF>
__device__ __forceinline__ void merge_slots_one_trip(const float* P, int ns, int lane, float& o0, float& o1,
                                                     float& L) {
  constexpr int D = 128;
  const float2 mlp = ld_partial2(P + (size_t)min(lane, ns - 1) * (D + 2) + D);
  const float ml = mlp.x, ll = mlp.y;
  float2 x[SF];
#pragma unroll
  for (int u = 0; u < SF; ++u) x[u] = ld_partial2(P + (size_t)min(u, ns - 1) * (D + 2) + 2 * lane);
  const bool mine = lane < ns && ml != NEG_INF;
  const float M = wmax(mine ? ml : NEG_INF);
  const float w = mine ? exp2f(ml - M) : 0.0f;
  L = wsum(mine ? ll * w : 0.0f);
#pragma unroll
  for (int u = 0; u < SF; ++u) {
    if (u < ns) {
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
      o0 = __builtin_fmaf(x[u].x, wu, o0);
      o1 = __builtin_fmaf(x[u].y, wu, o1);
    }
  }
}

// Merge and un-rotation of query heads hq0 .. hq0 + 3 (wave j merges head j,
// lane l dims 2 l and 2 l + 1).  Up to 32 slots: one round trip
// (merge_slots_one_trip), the R_V^T rows loaded beside the partials.  More slots (the small-batch shapes, many
// window blocks): three dependent steps whatever the count (up to 256):
// every slot's m and l of the four heads into shared memory in one round
// trip; per head (wave) the maximum, the sum and each slot's weight; then
// o' = sum of weight x o'_s with 32 slots' loads in flight per round trip;
// the R_V^T rows after that.
__device__ __forceinline__ void combine_group4(const CombineArgs& a, int b, int hq0, FusedSmem& S) {
  constexpr int D = 128, SB = 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ns = a.nslots;
  const float* P0 = a.partials + ((size_t)b * a.Hq + hq0) * a.pstride * (D + 2);
  const float* P = P0 + (size_t)wave * a.pstride * (D + 2);
  float o0 = 0.0f, o1 = 0.0f, L = 0.0f;
  RRows<D, 4> rr;
  if (ns <= 32) {
    if (!a.absorb_v) rr = load_r_rows<D, 4>(a.rvT);
    if (ns <= 8) merge_slots_one_trip<8>(P, ns, lane, o0, o1, L);
    else merge_slots_one_trip<32>(P, ns, lane, o0, o1, L);
  } else {
    static_assert(4 * 2 * kMaxSplits <= sizeof(S.scratch) / sizeof(float), "merge weights");
    float* wm = S.scratch;                // [4][ns]: m, then the slot weight
    float* wl = S.scratch + 4 * ns;       // [4][ns]: l
    for (int i = tid; i < 4 * ns; i += 256) {
      const int j = i / ns, sl = i - j * ns;
      const float* p = P0 + ((size_t)j * a.pstride + sl) * (D + 2);
      wm[i] = ld_partial<true>(p + D);
      wl[i] = ld_partial<true>(p + D + 1);
    }
    __syncthreads();
    float mx = NEG_INF;
    for (int sl = lane; sl < ns; sl += 64) mx = fmaxf(mx, wm[wave * ns + sl]);
    const float M = wmax(mx);
    float lsum = 0.0f;
    for (int sl = lane; sl < ns; sl += 64) {
      const float m = wm[wave * ns + sl];
      const float w = m == NEG_INF ? 0.0f : exp2f(m - M);
      lsum = __builtin_fmaf(wl[wave * ns + sl], w, lsum);
      wm[wave * ns + sl] = w;
    }
    L = wsum(lsum);
    wave_lds_sync();  // the wave's weights, written by its own lanes, are read below
    for (int s0 = 0; s0 < ns; s0 += SB) {
      float2 x[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) x[u] = ld_partial2(P + (size_t)min(s0 + u, ns - 1) * (D + 2) + 2 * lane);
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const float w = s0 + u < ns ? wm[wave * ns + s0 + u] : 0.0f;
        o0 = __builtin_fmaf(x[u].x, w, o0);
        o1 = __builtin_fmaf(x[u].y, w, o1);
      }
    }
    __syncthreads();                      // every wave is done with the weights (scratch is reused)
    if (!a.absorb_v) rr = load_r_rows<D, 4>(a.rvT);
  }
  const float inv = 1.0f / L;
  if (a.absorb_v) {                       // o' in the V-rotated basis
    store_out(a, ((size_t)b * a.Hq + hq0 + wave) * D + 2 * lane, o0 * inv);
    store_out(a, ((size_t)b * a.Hq + hq0 + wave) * D + 2 * lane + 1, o1 * inv);
    return;
  }
  float* os = S.scratch;                  // [4][128]
  float* part = S.scratch + 4 * D;        // [4 waves][4][128]
  os[wave * D + 2 * lane] = o0 * inv;
  os[wave * D + 2 * lane + 1] = o1 * inv;
  __syncthreads();
  rotate_rows_regs<D, 4, 4>(os, rr, part);
  __syncthreads();
  for (int idx = tid; idx < 4 * D; idx += 256) {
    const int j = idx >> 7, d = idx & 127;
    store_out(a, ((size_t)b * a.Hq + hq0 + j) * D + d, rot_sum<D, 4, 4>(part, j, d));
  }
  __syncthreads();                        // os / part are rewritten by the next group
}

// fp32 published q of one head group into shared memory (window blocks).
__device__ void load_published_q(const DecodeArgs& a, int pidx, FusedSmem& S) {
  const float* src = a.qpub + (size_t)pidx * kQPub;
  for (int i = threadIdx.x; i < 4 * 128; i += blockDim.x) S.qs[i >> 7][i & 127] = ld_partial<true>(src + i);
  if (threadIdx.x < 4) {
    S.qsum[threadIdx.x] = ld_partial<true>(src + 512 + threadIdx.x);
    S.qeq[threadIdx.x] = __float_as_int(ld_partial<true>(src + 516 + threadIdx.x));
  }
  __syncthreads();
}

// q of head group g of a window block into shared memory (S.qs, S.qsum,
// S.qeq): SELF, rotated by the block itself (R_K rows and the raw q in one
// round trip); else from the record of the prologue launch.
template <bool SELF>
__device__ inline void window_q_group(const DecodeArgs& a, int bh, int g, FusedSmem& S) {
  if constexpr (SELF) {
    const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
    const QRotLoads ql = q_rotation_loads(a, b, h * 4 * a.G + 4 * g);
    q_rotation_finish(a, ql, S);
  } else {
    load_published_q(a, bh * a.G + g, S);
  }
}

// Row loads of one 64-token pass of a window block: the K pieces a thread
// scores (token tid/4, dims 32 (tid%4) .. +32) and the V pieces it
// accumulates (tokens tid/16 + 16 i, dims 8 (tid%16) .. +8); slots past the
// pass are zero.
struct WinRows {
  uint4 k[4];
  uint4 v[4];
};

__device__ inline int window_len(const SeqView& sv) {
  return (sv.win.b0 - sv.win.a0) + (sv.win.b1 - sv.win.a1);
}

__device__ inline WinRows window_rows(const DecodeArgs& a, const SeqView& sv, int bh, int vt0, int v_hi) {
  const int tid = threadIdx.x, n = min(64, v_hi - vt0);
  WinRows r;
  const int tok = tid >> 2, part = tid & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.k[i] = make_uint4(0, 0, 0, 0);
  if (tok < n) {
    const uint4* rp = reinterpret_cast<const uint4*>(win_row(a, sv, a.k, bh, win_token(sv.win, vt0 + tok)) + 32 * part);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.k[i] = rp[i];
  }
  const int g = tid >> 4, c = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tk = g + 16 * i;
    r.v[i] = make_uint4(0, 0, 0, 0);
    if (tk < n) r.v[i] = *reinterpret_cast<const uint4*>(win_row(a, sv, a.v, bh, win_token(sv.win, vt0 + tk)) + 8 * c);
  }
  return r;
}

// The block's first pass of rows, issued before it waits for q.
__device__ inline WinRows window_first_rows(const DecodeArgs& a, const SeqView& sv, int bh, int wblk) {
  const int v_lo = wblk * sv.win.chunk;
  return window_rows(a, sv, bh, v_lo, min(window_len(sv), v_lo + sv.win.chunk));
}

// bf16 window tokens (sink + recent) of one (sequence, kv head), up to
// win.chunk of them in 64-token passes with fp32 VALU arithmetic, for each
// head group of 4 query heads in turn.  first: the first pass's rows, already
// issued (later passes, and the passes of later groups, load theirs at their
// start; a later group loads its first pass's rows again, from cache, rather
// than hold them in registers).  q: window_q_group.
__device__ __forceinline__ void window_group(const DecodeArgs& a, const SeqView& sv, int bh, int b, int hq0, int wblk,
                                             FusedSmem& S, const WinRows& first);

template <int G, bool SELF>
__device__ void window_block(const DecodeArgs& a, const SeqView& sv, int bh, int b, int h, int wblk, FusedSmem& S,
                             const WinRows& first) {
  window_q_group<SELF>(a, bh, 0, S);
  window_group(a, sv, bh, b, h * 4 * G, wblk, S, first);
#pragma unroll
  for (int g = 1; g < G; ++g) {
    __syncthreads();                  // shared memory is reused by the next group
    const WinRows again = window_first_rows(a, sv, bh, wblk);
    window_q_group<SELF>(a, bh, g, S);
    window_group(a, sv, bh, b, h * 4 * G + 4 * g, wblk, S, again);
  }
}

__device__ __forceinline__ void window_group(const DecodeArgs& a, const SeqView& sv, int bh, int b, int hq0, int wblk,
                                             FusedSmem& S, const WinRows& first) {
  constexpr int D = 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int len = window_len(sv);
  const int v_lo = wblk * sv.win.chunk;
  const int v_hi = min(len, v_lo + sv.win.chunk);
  float* sc = S.scratch;               // [4][64]
  float* wm = S.scratch + 256;         // [4] running max
  float* wl = S.scratch + 260;         // [4] running sum
  float* wa = S.scratch + 264;         // [4] rescale factor
  float* red = S.scratch + 272;        // [4 waves][4][128]
  if (tid < 4) {
    wm[tid] = NEG_INF;
    wl[tid] = 0.0f;
  }
  const int g = tid >> 4, c = tid & 15;      // PV role: token group, 8-dim chunk
  float o[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) o[j][k] = 0.0f;
  __syncthreads();
  WinRows cur = first;
  for (int vt0 = v_lo; vt0 < v_hi; vt0 += 64) {
    const int n = min(64, v_hi - vt0);
    if (vt0 != v_lo) cur = window_rows(a, sv, bh, vt0, v_hi);
    {  // scores: 4 lanes per token, 32 dims each
      const int tok = tid >> 2, part = tid & 3;
      float dots[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tok < n) {
        const uint4 us[4] = {cur.k[0], cur.k[1], cur.k[2], cur.k[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x[8];
          bf16x8(us[i], x);
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) dots[j] = __builtin_fmaf(S.qs[j][32 * part + 8 * i + k], x[k], dots[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dots[j] += __shfl_xor(dots[j], 1);
        dots[j] += __shfl_xor(dots[j], 2);
      }
      if (part == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j * 64 + tok] = tok < n ? dots[j] : NEG_INF;
    }
    __syncthreads();
    {  // online softmax update, one wave per head
      const float sv = sc[wave * 64 + lane];
      const float mold = wm[wave];
      const float mnew = fmaxf(mold, wmax(sv));
      const float p = (sv == NEG_INF) ? 0.0f : exp2f(sv - mnew);
      const float l = wsum(p);
      sc[wave * 64 + lane] = p;
      if (lane == 0) {
        const float alpha = (mold == NEG_INF) ? 0.0f : exp2f(mold - mnew);
        wa[wave] = alpha;
        wm[wave] = mnew;
        wl[wave] = wl[wave] * alpha + l;
      }
    }
    __syncthreads();
    {  // PV: thread (g, c) over tokens g, g+16, g+32, g+48 of the tile
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float al = wa[j];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[j][k] *= al;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = g + 16 * i;
        if (tok < n) {
          float x[8];
          bf16x8(cur.v[i], x);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = sc[j * 64 + tok];
#pragma unroll
            for (int k = 0; k < 8; ++k) o[j][k] = __builtin_fmaf(p, x[k], o[j][k]);
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[j][k] += __shfl_xor(o[j][k], 16);
      o[j][k] += __shfl_xor(o[j][k], 32);
    }
  if (lane < 16)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) red[(wave * 4 + j) * D + 8 * c + k] = o[j][k];
  __syncthreads();
  const int slot = a.win.slot0 + wblk;
  for (int idx = tid; idx < 4 * D; idx += 256) {
    const int j = idx >> 7, d = idx & 127;
    float* dst = a.partials + (((size_t)b * a.Hq + hq0 + j) * a.pstride + slot) * (D + 2);
    st_partial(dst + d, ((red[j * D + d] + red[(4 + j) * D + d]) + red[(8 + j) * D + d]) + red[(12 + j) * D + d]);
    if (d == 0) {
      st_partial(dst + D, wm[j]);
      st_partial(dst + D + 1, wl[j]);
    }
  }
}

// Reductions over the 16 lanes of one query head (lanes with equal lane % 4):
// rotations by 4 and 8 inside each 16-lane row, then the gfx950 row swaps.
template <int CTRL>
__device__ inline float dpp_row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ inline float head_max(float v) {
  v = fmaxf(v, dpp_row_ror<0x124>(v));     // row_ror:4
  v = fmaxf(v, dpp_row_ror<0x128>(v));     // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float head_sum(float v) {
  v += dpp_row_ror<0x124>(v);
  v += dpp_row_ror<0x128>(v);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct TileRegs {
  u4 k0, k1;   // K codes of token tile + lane (32 bytes)
  u4 km, vm;   // K and V scale|zero of tokens tile + 4 blk .. + 3
  u4 v0, v1;   // V code record of this lane (32 bytes)
};

// The four INT2 streams of one (sequence, kv head) as buffer resources: the
// plane base is uniform (scalar registers), each lane adds a fixed 32-bit
// offset and each tile a uniform one, so no 64-bit address arithmetic runs per
// tile.  A resource covers exactly that (sequence, kv head)'s part of the plane.
struct TileStreams {
  __amdgpu_buffer_rsrc_t kc;   // K codes, 32 bytes per token
  __amdgpu_buffer_rsrc_t km;   // K scale|zero, 4 bytes per token
  __amdgpu_buffer_rsrc_t vm;   // V scale|zero
  __amdgpu_buffer_rsrc_t vc;   // V code tiles, 2 KiB per 64 tokens (32 bytes per token)
};

constexpr int kBufferConfig = 0x00020000;   // raw 32-bit data, no swizzle (gfx9 family)

// Cache policy bits of a buffer load: nt (every code byte is read once per
// launch).
constexpr int kStreamOnce = 2;

__device__ inline __amdgpu_buffer_rsrc_t plane_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferConfig);
}

__device__ inline TileStreams tile_streams(const DecodeArgs& a, int bh) {
  constexpr int D = 128;
  TileStreams s;
  s.kc = plane_rsrc(a.k.codes + kcode_byte(bh, a.cap, 0, 0, D), a.cap * 32);
  s.km = plane_rsrc(a.k.meta + meta_index(bh, a.cap, 0, 0, D), a.cap * 4);
  s.vm = plane_rsrc(a.v.meta + meta_index(bh, a.cap, 0, 0, D), a.cap * 4);
  s.vc = plane_rsrc(a.v.codes + (size_t)bh * (a.cap / kTile) * 2048, a.cap * 32);
  return s;
}


// ---------------------------------------------------------------------------
// INT2 splits of the head_dim-128 attention kernel on v_mfma_f32_16x16x32_f16
// ---------------------------------------------------------------------------
//
// Lane l = 16 g + c (c = l % 16, g = l / 16).  The columns of both products
// are head pieces: column c is query head 4 grp + j of the kv head (grp =
// (c / 4) % 2, j = c % 4) as piece c / 8 (0: hi = fp16(x), 1: lo =
// fp16(x - hi)); with 4 query heads per kv head the columns of grp 1 are zero.
// The two pieces of an operand thus ride in columns that would otherwise be
// padding.
//
// QK^T, per 64-token tile: 4 token blocks tb x 4 dim chunks kc.  Row r of
// token block tb is token tau(tb, r) = 32 (tb/2) + 8 (r/4) + 4 (tb%2) + r%4 of
// the tile.  A (lane (r, g)) = 8 codes of that token: code word 2 g + kc/2 of
// its row, bytes 0 and 2 (even kc) or 1 and 3 (odd kc); item 2d + e is the
// code at bit pair d of the e-th of those bytes, as the fp16 denormal
// c 4^d 2^-24.  B (lane (c, g)) = the same dims of column c's q times
// 2^(eq - 2d).  Output: lane (c, g) register i = dot of column c with token
// tau(tb, 4 g + i).  Columns c and c + 8 (the pieces of one head) are added by
// a row rotation; both lanes then hold the head's dot.
//
// PV, per tile: 2 token chunks tc x 8 dim blocks db.  K slot (g, i) of chunk
// tc is token 32 tc + 8 g + i = tau(2 tc + i/4, 4 g + i%4): the very tokens
// whose scores lane (c, g) holds, so B (lane (c, g)) = column c's piece of
// s_V p for its own 8 tokens, with no data movement.  A (lane (r, g)) = the
// codes of dim 16 db + r for those tokens: in the V tile, lane record
// r + 16 (db % 4), word 4 tc + g, bytes 0 and 2 (db < 4) or 1 and 3; item i
// sits at bit pair i/2, a factor 4^(i/2) that the weight carries as 4^-(i/2).
// Output: lane (c, g) register i = dim 16 db + 4 g + i of column c.

// 8 codes of a code word as a 16x16x32 operand: bytes (0, 2) for hf = 0 or
// (1, 3) for hf = 1; dword d = bit pair d of both bytes (items 2d, 2d + 1).
__device__ inline h8 codes8(uint32_t w, int hf) {
  const uint32_t u = hf ? (w >> 8) : w;
  const u4 v = {u & 0x00030003u, u & 0x000C000Cu, u & 0x00300030u, u & 0x00C000C0u};
  return __builtin_bit_cast(h8, v);
}

// v plus the value of the lane 8 away within its row of 16 (lanes c and c + 8
// both get the sum): one add with a row rotation on its source.
__device__ inline float row_add8(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
}
// Maximum and sum over the four lane groups (lanes c, c + 16, c + 32, c + 48).
__device__ inline float groups_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float groups_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row rotation by 4 within each row of 16, added: lane c gets v_c + v_(c+4 mod 16).
__device__ inline float row_add4(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true));
}
__device__ inline float row_max4(float v) {
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true)));
}

// Four query heads per kv head (G = 1) use the K dimension of the QK^T product
// for two token sets instead: k slots 0-15 (lane groups 0, 1) carry the dims
// of row r's token of set A, slots 16-31 those of set B, and each column's q
// fills only the slots of its own set (the other half is zero).  Column c is
// then head j = c % 4 of set (c / 4) % 2 as piece c / 8, every lane's scores
// are real (none belong to a zero column), and a tile is 2 token pairs tp x 8
// instructions of 16 dims (word w' = 4 (g % 2) + wp of the token's code row,
// half h).  Rows: token 32 set + 8 (r / 4) + 4 tp + r % 4.  Output: lane
// (c, g) register i = token 32 set + 8 g + 4 tp + i of its column.  PV per
// set: K slot (g, i) = token 32 set + 8 g + i, i = 4 tp + register, the
// lane's own weights for the columns of that set and zero for the others;
// the sets and the pieces are added after the tile loop.
template <bool KS>
struct Tile16 {
  u4 kq[KS ? 2 : 1];       // KS: the 16-byte chunk g % 2 of the row of token pair tp's token
  uint2 k[KS ? 1 : 4];     // plain: code words 2 g, 2 g + 1 of token tau(tb, c)
  uint32_t v[4][2];        // V record words g and 4 + g of records c + 16 q
  uint32_t km, vm;         // scale|zero of token t0 + lane (K, V)
};

// Loads of one tile for one lane; the scale|zero words are exchanged through
// shared memory by the wave.
template <bool KS>
__device__ inline Tile16<KS> load_tile16(const TileStreams& st, int t0, int koff, int voff, int moff) {
  Tile16<KS> r;
  const int oc = t0 * 32, om = t0 * 4;
  // in order of first use: the scale|zero words, the K codes, the V codes
  r.km = __builtin_amdgcn_raw_buffer_load_b32(st.km, moff, om, 0);
  r.vm = __builtin_amdgcn_raw_buffer_load_b32(st.vm, moff, om, 0);
  __builtin_amdgcn_sched_barrier(0);    // keeps the issue order (loads return in it)
  if constexpr (KS) {
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) r.kq[tp] = __builtin_amdgcn_raw_buffer_load_b128(st.kc, koff + 64 * tp, oc, kStreamOnce);
  } else {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      r.k[tb] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                              st.kc, koff + 512 * (tb >> 1) + 64 * (tb & 1), oc, kStreamOnce));
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      r.v[q][hf] = __builtin_amdgcn_raw_buffer_load_b32(st.vc, voff + 256 * q + 1024 * hf, oc, kStreamOnce);
  return r;
}

// One INT2 split of the head_dim-128 attention kernel (G head groups of 4 query heads).
template <int G, bool SELF>
__device__ void int2_split16(const DecodeArgs& a, const SeqView& sv, int b, int h, int bh, int split,
                             FusedSmem& S) {
  constexpr int D = 128, WPB = 4;
  constexpr bool KS = G == 1;                     // token sets in the K dimension
  constexpr int NOP = KS ? 8 : 4;                 // q operands per lane
  // wave index as a uniform value: the tile loop is controlled by scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int jh = c & 3, piece = c >> 3;
  const int grp = KS ? 0 : (c >> 2) & 1;          // head group of the column
  const int set = KS ? (c >> 2) & 1 : 0;          // token set of the column (KS)
  const int lo = a.plan.a0, hi = sv.hi;          // INT2 token range (empty in a short sequence)
  const int tile_first = lo >> 6;
  const int ntiles = hi > lo ? ((hi - 1) >> 6) - tile_first + 1 : 0;
  // Split s covers tiles [start(s), start(s + 1)): equal shares of the range
  // (one round: the host's shares)
  auto split_start = [&](int s) -> int {
    const int Sn = a.plan.splits;
    if (s >= Sn) return ntiles;
    if (a.one_round) return min(ntiles, (int)(a.share[s] * (float)ntiles));
    return s * ntiles / Sn;
  };
  const int s_t0 = split_start(split);
  const int s_t1 = split_start(split + 1);
  const int t_last = max(s_t1 - 1, 0);            // a valid tile for clamped loads
  const int ti0 = s_t0 + wave;
  const TileStreams st = tile_streams(a, bh);
  auto tile_t0 = [&](int ti) { return (tile_first + ti) << 6; };
  // lane parts of the load offsets (the per-token-block and per-record parts
  // are constants)
  const int koff = KS ? (g & 1) * 1024 + 16 * (32 * (g >> 1) + 8 * (c >> 2) + (c & 3))
                      : (g >> 1) * 1024 + 8 * (g & 1) + 16 * (8 * (c >> 2) + (c & 3));
  const int voff = 16 * c + 4 * g;
  const int moff = 4 * lane;
  // first of the 4 tokens (of the tile) whose scores register block tb / tp holds
  auto tok_of = [&](int t) { return KS ? 32 * set + 8 * g + 4 * t : 32 * (t >> 1) + 8 * g + 4 * (t & 1); };

  // q operands of this lane's column, in shared memory (every wave has the
  // same ones; they would otherwise hold NOP x 4 registers through the tile
  // loop), read per tile.  Operand n (32 dims: lane group gp, chunk kc) is
  // taken as: plain, n = kc, gp = the lane's group; KS, instruction (wp, h) =
  // n / 2, n % 2 takes lane group 2 (g % 2) + wp / 2, chunk 2 (wp % 2) + h,
  // zero unless the column's set is the lane's (g / 2).
  auto hq_of = [&](int gg) { return h * 4 * G + 4 * gg; };   // first query head of group gg
  auto op_src = [&](int n, int lg, int& gp, int& kc) {
    if (KS) {
      const int wp = n >> 1, hh = n & 1;
      gp = 2 * (lg & 1) + (wp >> 1);
      kc = 2 * (wp & 1) + hh;
    } else {
      gp = lg;
      kc = n;
    }
  };
  const float pm = (float)piece;                  // 1 in the lanes of low pieces
  float qsum = 0.0f;
  int eq = 0;
  float vmax;
  Tile16<KS> r[kDepth16];
  if constexpr (SELF) {
    // The block rotates q itself.  The V scale maximum as it stood before
    // this launch (a step's append folds its token's scale in at the end of
    // the launch: every INT2 token was appended earlier), the rotation's loads
    // (R_K rows, the raw q), the first tile (the appended token lies at least
    // a tile past the INT2 range), the rotation while that tile is in flight,
    // the other tiles, then each head group's operands.
    vmax = a.v.smax[bh];
    QRotLoads ql = q_rotation_loads(a, b, hq_of(0));
    r[0] = load_tile16<KS>(st, tile_t0(min(ti0, t_last)), koff, voff, moff);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      if (gg == 1) {                              // group 1's raw q (R_K rows as for group 0)
        const uint16_t* qb = a.q + ((size_t)b * a.Hq + hq_of(1)) * D;
        ql.q0 = bf16_to_f32(qb[threadIdx.x]);
        ql.q1 = bf16_to_f32(qb[threadIdx.x + 256]);
        __syncthreads();                          // group 0's operands are written
      }
      q_rotation_finish(a, ql, S);                // S.qs, S.qsum, S.qeq of group gg
      if (gg == G - 1) {
        // the R rows are dead: the other tiles go out before the operands
#pragma unroll
        for (int k = 1; k < kDepth16; ++k) {
          r[k] = load_tile16<KS>(st, tile_t0(min(ti0 + k * WPB, t_last)), koff, voff, moff);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (grp == gg) {
        qsum = S.qsum[jh];
        eq = S.qeq[jh];
      }
      // the group's 512 distinct operand words (the record's layout: word
      // 16 ((piece 4 + lane group) 4 + head) + 4 chunk + d), each formed once,
      // then every lane's copies of them
      uint32_t* stage = reinterpret_cast<uint32_t*>(S.scratch);   // free after the rotation
      for (int i = threadIdx.x; i < 512; i += 64 * WPB) {
        const int v = i >> 4, wd = i & 15;
        stage[i] = q_operand16_pair(S, v & 3, (v >> 2) & 3, v >> 4, wd >> 2, wd & 3);
      }
      __syncthreads();
      for (int e = threadIdx.x; e < NOP * 64; e += 64 * WPB) {
        const int n = e >> 6, l = e & 63, lc = l & 15, lg = l >> 4;
        if ((KS ? 0 : (lc >> 2) & 1) != gg) continue;
        u4 w = {0u, 0u, 0u, 0u};
        if (!KS || ((lc >> 2) & 1) == (lg >> 1)) {
          int gp, kc;
          op_src(n, lg, gp, kc);
          w = *reinterpret_cast<const u4*>(stage + 16 * (((lc >> 3) * 4 + gp) * 4 + (lc & 3)) + 4 * kc);
        }
        S.qops[n][l] = w;
      }
    }
  } else {
    // q from the record the prologue launch wrote, first: it comes back from
    // cache ahead of the tiles, and the loads return in issue order, so the
    // first tile's work waits for q and that tile only
    h8 qop[NOP];
#pragma unroll
    for (int n = 0; n < NOP; ++n) qop[n] = h8{0, 0, 0, 0, 0, 0, 0, 0};
    const __amdgpu_buffer_rsrc_t qr = plane_rsrc(a.qpub + (size_t)(bh * G + grp) * kQPub, kQPub * 4);
    if ((!KS || set == (g >> 1)) && wave == 0) {
#pragma unroll
      for (int n = 0; n < NOP; ++n) {
        int gp, kc;
        op_src(n, g, gp, kc);
        const int vb = (kQPub16 + 16 * ((piece * 4 + gp) * 4 + jh) + 4 * kc) * 4;
        qop[n] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(qr, vb, 0, 0));
      }
    }
    qsum = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, (512 + jh) * 4, 0, 0));
    eq = (int)__builtin_amdgcn_raw_buffer_load_b32(qr, (516 + jh) * 4, 0, 0);
    vmax = a.v.smax[bh];
#pragma unroll
    for (int k = 0; k < kDepth16; ++k) {
      r[k] = load_tile16<KS>(st, tile_t0(min(ti0 + k * WPB, t_last)), koff, voff, moff);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (wave == 0) {
#pragma unroll
      for (int n = 0; n < NOP; ++n) S.qops[n][lane] = __builtin_bit_cast(u4, qop[n]);
    }
  }
  __syncthreads();
  const u4* qop_lds = &S.qops[0][lane];
  // z: an offset of zero that the compiler cannot see through, taken once
  // per tile, so that the operand reads stay in the tile loop instead of
  // being hoisted into registers
  auto qop_at = [&](int n, int z) { return __builtin_bit_cast(h8, qop_lds[n * 64 + z]); };
  const float cK = ldexpf(1.0f, 24 - eq);         // undoes 2^eq and the 2^-24 code scale
  const float zq = ldexpf(qsum, eq - 24);         // sum(q_rot) in units of the raw dot
  int ev2 = 0;
  if (vmax > 0.0f) frexpf(vmax, &ev2);
  // s_V * 2^ev < 2^15; capped so that p * 2^ev and its sums stay far from fp32
  // overflow (a cap that binds only for V scales below 2^-45)
  const int ev = (vmax > 0.0f) ? min(15 - ev2, 60) : 0;
  const float cV = ldexpf(1.0f, 24 - ev);
  // The softmax weight p of a token is computed as p' = p 2^(ev - 2s), s = the
  // bit pair of its V code (2 (tb % 2) + i / 2 for register i of token block
  // tb; 2 tp + i / 2 with token sets), so that s_V p' is the PV operand as it
  // stands.  l and sum(p z_V) are kept per s and brought back at the end.
  f4 ao[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) ao[db] = f4{0, 0, 0, 0};
  float m = NEG_INF, ls[4], pz[4], cs[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ls[s] = pz[s] = cs[s] = 0.0f;
  uint32_t* msm = S.meta16[wave];                 // [0, 64) K, [64, 128) V scale|zero of the tile
  constexpr int NB = KS ? 2 : 4;                  // register blocks of scores (tp or tb)
  // The tile loop starts with only its own tiles in flight, in the order it
  // consumes them, and each use waits for exactly the oldest one.

  // EDGE: the tile crosses the split's INT2 range [lo, hi) (its first or last
  // tile): tokens outside it get no weight.  A separate instantiation keeps
  // the masks out of the other tiles.
  auto process = [&](const Tile16<KS>& cur, int t0, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const bool edge = t0 < lo || t0 + 64 > hi;
    msm[lane] = cur.km;
    msm[64 + lane] = cur.vm;
    f4 acc[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) acc[rb] = f4{0, 0, 0, 0};
    // one operand read per instruction column, used by every register block;
    // the reads run two operands ahead of their use
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    h8 qbuf[NOP];
    qbuf[0] = qop_at(0, z);
    qbuf[1] = qop_at(1, z);
#pragma unroll
    for (int n = 0; n < NOP; ++n) {
      if (n + 2 < NOP) qbuf[n + 2] = qop_at(n + 2, z);
      const h8 qn = qbuf[n];
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        uint32_t w;
        if constexpr (KS) {
          const uint32_t kw[4] = {cur.kq[rb].x, cur.kq[rb].y, cur.kq[rb].z, cur.kq[rb].w};
          w = kw[n >> 1];
        } else {
          w = n < 2 ? cur.k[rb].x : cur.k[rb].y;
        }
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8(w, n & 1), qn, acc[rb], 0, 0, 0);
      }
    }
    // the lanes read each other's words: the wave's writes complete first
    wave_lds_sync();
    PHASE_FENCE();
    float u[NB][4];
    float tmax = NEG_INF;
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int tok = tok_of(rb);
      const u4 kmv = *reinterpret_cast<const u4*>(msm + tok);
      const uint32_t kmr[4] = {kmv.x, kmv.y, kmv.z, kmv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dot = row_add8(acc[rb][i]);   // hi + lo pieces
        // s_K * dot + z_K * sum(q), fp16 metadata read in place
        u[rb][i] = __builtin_fmaf(hi_half(kmr[i]), zq, __builtin_fmaf(lo_half(kmr[i]), dot, 0.0f));
        tmax = fmaxf(tmax, u[rb][i]);
      }
    }
    if (__builtin_expect(EDGE && edge, 0)) {
      tmax = NEG_INF;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if ((unsigned)(t0 + tok_of(rb) + i - lo) >= (unsigned)(hi - lo)) u[rb][i] = NEG_INF;
          tmax = fmaxf(tmax, u[rb][i]);
        }
    }
    tmax *= cK;
    // the head's maximum is only needed when some score exceeds its running
    // maximum (every lane of a head holds that maximum)
    if (__any(tmax > m)) {
      const float mnew = fmaxf(m, groups_max(KS ? row_max4(tmax) : tmax));
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ls[s] *= alpha;
        pz[s] *= alpha;
        cs[s] = (float)(ev - 2 * s) - mnew;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) ao[db] *= alpha;
      m = mnew;
    }
    h8 pw[2];                                      // this column's piece of s_V p' (KS: of its set)
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const u4 vmv = *reinterpret_cast<const u4*>(msm + 64 + tok_of(rb));
      const uint32_t vmr[4] = {vmv.x, vmv.y, vmv.z, vmv.w};
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = KS ? 2 * rb + (i >> 1) : 2 * (rb & 1) + (i >> 1);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(cK, u[rb][i], cs[s]));
        ls[s] += p;
        pz[s] = __builtin_fmaf(p, hi_half(vmr[i]), pz[s]);
        x[i] = __builtin_fmaf(lo_half(vmr[i]), p, 0.0f);   // s_V p' (fp16 scale read in place)
      }
      // this column's piece, two values at a time: hi = fp16(x); the low
      // piece's lanes (pm = 1) take fp16(x - hi) instead
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const _Float16 h0 = (_Float16)x[i], h1 = (_Float16)x[i + 1];
        const float y0 = __builtin_fmaf(-(float)h0, pm, x[i]);
        const float y1 = __builtin_fmaf(-(float)h1, pm, x[i + 1]);
        const int e = KS ? 4 * rb + i : 4 * (rb & 1) + i;
        pw[KS ? 0 : rb >> 1][e] = (_Float16)y0;
        pw[KS ? 0 : rb >> 1][e + 1] = (_Float16)y1;
      }
    }
    PHASE_FENCE();
    if constexpr (KS) {
      const h8 zero = h8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const h8 op = set == s2 ? pw[0] : zero;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          ao[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8(cur.v[db & 3][s2], db >> 2), op, ao[db], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int tc = 0; tc < 2; ++tc)
#pragma unroll
        for (int db = 0; db < 8; ++db)
          ao[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8(cur.v[db & 3][tc], db >> 2), pw[tc], ao[db], 0, 0, 0);
    }
  };

  // The wave's tiles are ti0 + WPB i, i < n; r[i % kDepth16] holds tile i.
  // Every processed register set is reloaded at once with the tile kDepth16
  // ahead, so the same loads are in flight on every path through the loop
  // (kDepth16 tiles, oldest first) and each use waits for exactly its own
  // loads; past the last tile the loads go through resources of zero length,
  // which return zeros without touching memory.
  const int n = s_t1 > ti0 ? (s_t1 - ti0 + WPB - 1) / WPB : 0;
  auto tile_of = [&](int i) { return tile_t0(ti0 + WPB * i); };
  TileStreams none = st;
  none.kc = plane_rsrc(a.k.codes, 0);
  none.km = plane_rsrc(a.k.meta, 0);
  none.vm = plane_rsrc(a.v.meta, 0);
  none.vc = plane_rsrc(a.v.codes, 0);
  // Rounds of kDepth16 tiles whose middle has no exit (a missing tile is
  // skipped, its reload still issued), so every path reaches the loop head
  // with the same loads in flight in the same order, and the first tile of a
  // round waits for its own loads only.
  for (int i = 0; i < n; i += kDepth16) {
#pragma unroll
    for (int k = 0; k < kDepth16; ++k) {
      if (i + k < n) process(r[k], tile_of(i + k), std::true_type{});
      r[k] = load_tile16<KS>(i + k + kDepth16 < n ? st : none, tile_of(min(i + k + kDepth16, n - 1)), koff, voff,
                             moff);
    }
  }

  // pieces of PV added (lanes c and c + 8), with token sets also the two sets
  // (lanes c and c + 4); l and sum(p z_V) over the lanes of the head, in true
  // units
  float lt = 0.0f, pzt = 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    lt = __builtin_fmaf(ldexpf(ls[s], 2 * s - ev), 1.0f, lt);
    pzt = __builtin_fmaf(ldexpf(pz[s], 2 * s - ev), 1.0f, pzt);
  }
  if constexpr (KS) {
    lt = row_add4(lt);
    pzt = row_add4(pzt);
  }
  lt = groups_sum(lt);
  pzt = groups_sum(pzt);
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ao[db][i] = row_add8(ao[db][i]);
      if constexpr (KS) ao[db][i] = row_add4(ao[db][i]);
    }

  static_assert(8 * WPB + WPB * 4 * D <= sizeof(S.scratch) / sizeof(float), "epilogue scratch");
  float* sm = S.scratch;                 // [WPB][4]
  float* sl = S.scratch + 4 * WPB;       // [WPB][4]
  float* so = S.scratch + 8 * WPB;       // [WPB][4][D]
  const int slot = a.plan.slot0 + split;
  // lanes holding a head's totals: c < 4 (token sets), piece 0 of its group
  const bool writer = KS ? c < 4 : piece == 0;
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    __syncthreads();                     // every wave is past its tile loop / the previous group's merge
    if (writer && grp == gg) {
      if (g == 0) {
        sm[wave * 4 + jh] = m;
        sl[wave * 4 + jh] = lt;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) so[(wave * 4 + jh) * D + 16 * db + 4 * g + i] = __builtin_fmaf(ao[db][i], cV, pzt);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 4 * D; idx += 64 * WPB) {
      const int rr = idx / D, d = idx - rr * D;
      float M = NEG_INF;
#pragma unroll
      for (int w = 0; w < WPB; ++w) M = fmaxf(M, sm[w * 4 + rr]);
      float O = 0.0f, L = 0.0f;
      if (M != NEG_INF) {
#pragma unroll
        for (int w = 0; w < WPB; ++w) {
          const float sw = exp2f(sm[w * 4 + rr] - M);
          O = __builtin_fmaf(so[(w * 4 + rr) * D + d], sw, O);
          L = __builtin_fmaf(sl[w * 4 + rr], sw, L);
        }
      }
      float* dst = a.partials + (((size_t)b * a.Hq + hq_of(gg) + rr) * a.pstride + slot) * (D + 2);
      st_partial(dst + d, O);
      if (d == 0) {
        st_partial(dst + D, M);
        st_partial(dst + D + 1, L);
      }
    }
  }
}

// Window role.  SELF: in a decode step the block whose chunk holds the
// appended token (the last window position of the sequence) first appends it
// to K and V with the one-token append's code (R_K and R_V rows and both
// inputs in one round trip; the window rows with device-scope stores; the V
// scale goes to a pending slot, which the merging block folds into the
// running maximum), then loads its rows.  Every other window block issues its
// first pass's rows first thing.
template <int G, bool SELF>
__device__ __forceinline__ void window_role(const DecodeArgs& a, const SeqView& sv, int bh, int b, int h, int wblk,
                                            FusedSmem& S) {
  if constexpr (SELF) {
    const int first = wblk * sv.win.chunk;
    const bool newest = a.app_blocks > 0 && window_len(sv) - 1 >= first && window_len(sv) - 1 < first + sv.win.chunk;
    if (newest) {
      const int2 tr = append_range(a.app, b);
      const AppendOneLoads kl = append_one_loads(a.app, bh, false, tr.x, tr.x);
      const AppendOneLoads vl = append_one_loads(a.app, bh, true, tr.x, tr.x);
      append_one_finish<true>(a.app, bh, false, tr.x, tr.x, tr.y, kl, S.scratch, S.scratch + 128);
      __syncthreads();
      append_one_finish<true>(a.app, bh, true, tr.x, tr.x, tr.y, vl, S.scratch, S.scratch + 128);
      __builtin_amdgcn_s_waitcnt(0);            // the rows are written before any thread reads them
      __syncthreads();
    }
  }
  const WinRows rows = window_first_rows(a, sv, bh, wblk);
  window_block<G, SELF>(a, sv, bh, b, h, wblk, S, rows);
}

// The attention launch of head_dim 128.  G: head groups of 4 query heads per
// kv head (G = Hq / Hkv / 4); the INT2 splits serve every group in one pass
// over the tiles (int2_split16).  SELF: the launch is the whole call: every
// block rotates its q itself and a step's token is appended by the window
// block that holds it.  Else decode_prologue_kernel ran first (q records, the
// append).  No block waits for another; the last block of a (sequence, kv
// head) to finish merges.
template <int WPB, int G, bool ONE, bool SELF>
__global__ __launch_bounds__(64 * WPB)
__attribute__((amdgpu_waves_per_eu(kMfmaWavesPerEu, kMfmaWavesPerEu)))
void decode_mfma_kernel(DecodeArgs a) {
  // The set-up below reads these arguments one after another (the sequence's
  // length, then its token sets, then the block's role); naming them first
  // issues their scalar loads together, one round trip instead of several.
  asm volatile("" ::"s"(a.Hkv), "s"(a.lens), "s"(a.N), "s"(a.M), "s"(a.T), "s"(a.int2_lead), "s"(a.win_blocks),
               "s"(a.ring0));
  asm volatile("" ::"s"(a.plan.a0), "s"(a.plan.b0), "s"(a.plan.a1), "s"(a.plan.b1), "s"(a.plan.chunk),
               "s"(a.win.a0), "s"(a.win.b0), "s"(a.win.a1), "s"(a.win.b1), "s"(a.win.chunk));
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  __shared__ FusedSmem S;
  const int y = (int)blockIdx.y;
  const SeqView sv = seq_view(a, b);
  if constexpr (ONE) {
    // One round: block y is INT2 split y; blocks 1 .. win_blocks first take
    // window chunk y - 1.  The host sizes the INT2 shares so that every block
    // ends at about the same time.
    const int wblk = y - 1;
    if (wblk >= 0 && wblk < a.win_blocks) {
      window_role<G, SELF>(a, sv, bh, b, h, wblk, S);
      __syncthreads();                  // shared memory is reused below
    }
    int2_split16<G, SELF>(a, sv, b, h, bh, y, S);
    finish_block<G>(a, bh, S);
    return;
  }
  // Several rounds, in dispatch order: int2_lead INT2 splits, the win_blocks
  // bf16 window blocks, the remaining INT2 splits (the lead splits fill the
  // compute units first).
  const int lead = a.int2_lead;
  if (y >= lead && y < lead + a.win_blocks) {
    window_role<G, SELF>(a, sv, bh, b, h, y - lead, S);
    finish_block<G>(a, bh, S);
    return;
  }
  int2_split16<G, SELF>(a, sv, b, h, bh, y < lead ? y : y - a.win_blocks, S);
  finish_block<G>(a, bh, S);
}

// The first launch of a decode call at head_dim 128 when the attention launch
// does not rotate q itself: blocks y < G rotate head group y's q and write its
// record (fp32 q, sums, exponents, the fp16 operand pieces); blocks G and G +
// 1 append the step's token (K, V).  The attention launch that follows in
// stream order reads both and waits for nothing.
template <int G>
__global__ __launch_bounds__(256) void decode_prologue_kernel(DecodeArgs a) {
  __shared__ FusedSmem S;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const int y = (int)blockIdx.y;
  if (y < G) {
    const QRotLoads ql = q_rotation_loads(a, b, h * 4 * G + 4 * y);
    q_rotation_finish(a, ql, S);
    publish_q<false>(a, bh * G + y, S);
    return;
  }
  const int2 tr = append_range(a.app, b);
  append_block<128, 4, 1>(a.app, bh, y == G + 1, tr.x, tr.x + 1, tr.x, tr.y, S.scratch, S.scratch + 128);
}

// ---------------------------------------------------------------------------
// head_dim 512 (four 128-wide quantization groups per head), at most 4 query
// heads per kv head
// ---------------------------------------------------------------------------
//
// Three launches: wide_qrot_kernel rotates q and writes, per (sequence, kv
// head, 128-dim slice s), the record of the 128-dim path (fp32 q of the 4
// heads over the slice, per-head sums and exponents, fp16 matrix-core
// operands); decode_wide_kernel streams the INT2 range and the bf16 windows
// into split partials; combine_kernel merges them and undoes the V rotation.
// In decode_wide_kernel the four waves of a block share every 64-token tile
// and wave w owns dims [128 w, 128 w + 128) = quantization group w: its K and
// V code tiles, its scales, its part of the scores and of the output.  The
// four partial scores meet in shared memory once per tile.

// q rotation of one 128-dim slice s of the rotated q, all heads of a kv head
// (zero-padded to 4), published as the slice's record.
__device__ void wide_qrot_block(const DecodeArgs& a, int bh, int s, FusedSmem& S, float* qraw,
                                float (*parts)[4][128]) {
  constexpr int D = 512;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  for (int i = tid; i < 4 * D; i += 256) {
    const int j = i / D, e = i - j * D;
    qraw[i] = j < a.Gq ? bf16_to_f32(a.q[((size_t)b * a.Hq + h * a.Gq + j) * D + e]) : 0.0f;
  }
  __syncthreads();
  // wave w reduces over input dims e in [128 w, 128 w + 128)
  // dims 128 s + 2 lane, + 1
  float acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j][0] = acc[j][1] = 0.0f;
  rot_rows_cols2<4, D>(qraw, D, a.rk, wave * 128, 128 * s + 2 * lane, acc);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    parts[wave][j][2 * lane] = acc[j][0];
    parts[wave][j][2 * lane + 1] = acc[j][1];
  }
  __syncthreads();
  {
    const int j = wave;                // wave j finishes head j
    float v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = lane + 64 * i;
      v[i] = ((((parts[0][j][d] + parts[1][j][d]) + parts[2][j][d]) + parts[3][j][d]) + 0.0f) * a.scale_log2;
    }
    S.qs[j][lane] = v[0];
    S.qs[j][lane + 64] = v[1];
    const float sum = wsum(v[0] + v[1]);
    const float amax = wmax(fmaxf(fabsf(v[0]), fabsf(v[1])));
    int e2 = 0;
    if (amax > 0.0f) frexpf(amax, &e2);
    if (lane == 0) {
      S.qsum[j] = sum;
      S.qeq[j] = (amax > 0.0f) ? 15 - e2 : 0;
    }
  }
  __syncthreads();
  publish_q<true>(a, bh * 4 + s, S);
}

// Grid: (sequence x kv head, slice).
__global__ __launch_bounds__(256) void wide_qrot_kernel(DecodeArgs a) {
  __shared__ FusedSmem S;
  __shared__ float qraw[4 * 512];
  __shared__ float parts[4][4][128];
  wide_qrot_block(a, (int)blockIdx.x, (int)blockIdx.y, S, qraw, parts);
}

// The decode step's first launch at head_dim 512: blocks y < 4 write the q
// records (slice y), blocks 4 + 2 g + v append the new token's group g of K
// (v = 0) or V (v = 1).  The attention launch that follows reads both.
__global__ __launch_bounds__(256) void wide_prologue_kernel(DecodeArgs a) {
  __shared__ FusedSmem S;
  __shared__ float qraw[4 * 512];
  __shared__ float parts[4][4][128];
  const int y = (int)blockIdx.y;
  if (y < 4)
    wide_qrot_block(a, (int)blockIdx.x, y, S, qraw, parts);
  else
    append_slice_block(a.app, (int)blockIdx.x, ((y - 4) & 1) != 0, (y - 4) >> 1, qraw, &parts[0][0][0]);
}

struct WideSmem {
  f4 u[2][4][64];              // per-wave partial scores of a tile (two buffers)
  float4 q[4][4][16][2];       // window: q of [slice][head][dims 8c .. 8c + 7]
  float sc[4][4][32];          // window: [wave][head][token] partial scores
  float p[4][32];              // window: softmax weights [head][token]
  float pv[4][4][64];          // bf16-V splits: [wave][head][token] softmax weights of the tile
  float wm[4], wl[4], wa[4];   // window: running max, sum, rescale factor per head
  uint32_t qlo[4][256];        // INT2 splits: low pieces of slice w's q operands, as published
};

// q operands of one 128-dim slice record for this lane (lane group pp =
// lane / 16, head j = lane % 4): high pieces into registers, low pieces into
// the slice's shared copy (read back through the returned pointer after the
// caller's barrier).  The record was written by an earlier launch.
__device__ inline const uint2* wide_q_operands(const DecodeArgs& a, int rec, uint32_t* qlo_smem, h4 (&qv)[8],
                                               float& qsum, int& eq) {
  const int lane = threadIdx.x & 63, j = lane & 3;
  const __amdgpu_buffer_rsrc_t qr = plane_rsrc(a.qpub + (size_t)rec * kQPub, kQPub * 4);
  const int vbase = (kQPubOps + 16 * (4 * (lane >> 4) + j)) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u4 wv = __builtin_amdgcn_raw_buffer_load_b128(qr, vbase + 16 * i, 0, 0);
    qv[2 * i] = as_h4(wv.x, wv.y);
    qv[2 * i + 1] = as_h4(wv.z, wv.w);
  }
  qsum = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, (512 + j) * 4, 0, 0));
  eq = (int)__builtin_amdgcn_raw_buffer_load_b32(qr, (516 + j) * 4, 0, 0);
  const u4 lw = __builtin_amdgcn_raw_buffer_load_b128(qr, (kQPubLo + 4 * lane) * 4, 0, 0);
  *reinterpret_cast<u4*>(qlo_smem + 4 * lane) = lw;
  return reinterpret_cast<const uint2*>(qlo_smem + 16 * (4 * (lane >> 4) + j));
}

// bf16 window tokens of one (sequence, kv head) with fp32 VALU arithmetic, in
// 32-token passes.  Window blocks take chunks of win.chunk tokens of the sink
// segment [a0, b0) first, then of the recent segment [a1, b1), so a block
// reads rows of one plane only: consecutive sink rows, or consecutive ring
// slots from (ring0 + its first index) mod M.  Wave w owns dims [128 w,
// 128 w + 128); lane (tq, c) owns dims 8 c .. 8 c + 7 of that slice for
// tokens tq + 4 i of a pass, so every row load is contiguous across 16 lanes.
template <int NH, bool VB>
__device__ void wide_window_block(const DecodeArgs& a, int bh, int b, int h, int wblk, WideSmem& W) {
  constexpr int D = 512, PT = 32, RI = PT / 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tq = lane >> 4, c = lane & 15;
  // the sequence's own segments; the split into sink and ring blocks is the
  // launch's (that of the longest sequence)
  const SeqView sv = seq_view(a, b);
  const int len0 = sv.win.b0 - sv.win.a0, len1 = sv.win.b1 - sv.win.a1;
  const int nb0 = ((a.win.b0 - a.win.a0) + a.win.chunk - 1) / a.win.chunk;
  const bool ring = wblk >= nb0;
  const int i_lo = (ring ? wblk - nb0 : wblk) * a.win.chunk;
  const int i_hi = min(ring ? len1 : len0, i_lo + a.win.chunk);
  // first row of the block and the plane's rows (elements): sink row a0 + i,
  // or ring slot (ring0 + i) mod M
  const int rows = ring ? a.M : a.N;
  const int nbytes = rows * D * 2;
  // the block's plane rows as buffer resources: a load at offset nbytes (past
  // them) returns zero
  const __amdgpu_buffer_rsrc_t kp =
      plane_rsrc(ring ? a.k.ring + row_offset(bh, a.M, 0, D) : a.k.sink + row_offset(bh, a.N, 0, D), nbytes);
  // V kept bf16 (VB): rows of the full plane by position (a.cap rows)
  const __amdgpu_buffer_rsrc_t vp =
      VB ? plane_rsrc(a.v.full + row_offset(bh, a.cap, 0, D), a.cap * D * 2)
         : plane_rsrc(ring ? a.v.ring + row_offset(bh, a.M, 0, D) : a.v.sink + row_offset(bh, a.N, 0, D), nbytes);
  const int pos0 = ring ? sv.win.a1 + i_lo : sv.win.a0 + i_lo;   // position of the block's first token
  int row0 = ring ? sv.ring0 + i_lo : sv.win.a0 + i_lo;
  if (row0 >= rows) row0 -= rows;
  const int col = 128 * wave + 8 * c;
  // q of the slice (4 heads, fp32 x scale * log2 e) into shared memory; read
  // back at each use, through an offset the compiler cannot see as constant,
  // so that it is not held in registers across the pass
  if (lane < 8 * NH) {
    const float* rec = a.qpub + (size_t)(bh * 4 + wave) * kQPub;
    const int j = lane >> 3, cc = 2 * (lane & 7);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        W.q[wave][j][cc + e][hf] = *reinterpret_cast<const float4*>(rec + j * 128 + 8 * (cc + e) + 4 * hf);
  }
  if (tid < 4) {
    W.wm[tid] = NEG_INF;
    W.wl[tid] = 0.0f;
  }
  float o[NH][8];
#pragma unroll
  for (int j = 0; j < NH; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) o[j][k] = 0.0f;
  __syncthreads();
  for (int p0 = i_lo; p0 < i_hi; p0 += PT) {
    const int n = min(PT, i_hi - p0);
    // byte offset of this lane's row i of the pass (nbytes, so loaded as
    // zero, for rows past the pass); rows wrap at most once
    auto roff = [&](int i) -> int {
      int r = row0 + (p0 - i_lo) + tq + 4 * i;
      if (r >= rows) r -= rows;
      return (tq + 4 * i < n) ? (r * D + col) * 2 : nbytes;
    };
    {  // partial scores of this slice
      u4 kr[RI];
#pragma unroll
      for (int i = 0; i < RI; ++i) kr[i] = __builtin_amdgcn_raw_buffer_load_b128(kp, roff(i), 0, 0);
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        float x[8];
        bf16x8(kr[i], x);
        int qc = c;
        asm volatile("" : "+v"(qc));
        float dots[NH];
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float4 q0 = W.q[wave][j][qc][0], q1 = W.q[wave][j][qc][1];
          const float qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
          dots[j] = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) dots[j] = __builtin_fmaf(qq[k], x[k], dots[j]);
        }
#pragma unroll
        for (int j = 0; j < NH; ++j) {   // sum over the 16 lanes of the row (rotations by 8, 4, 2, 1)
          dots[j] += dpp_row_ror<0x128>(dots[j]);
          dots[j] += dpp_row_ror<0x124>(dots[j]);
          dots[j] += dpp_row_ror<0x122>(dots[j]);
          dots[j] += dpp_row_ror<0x121>(dots[j]);
        }
        if (c == 0)
#pragma unroll
          for (int j = 0; j < NH; ++j) W.sc[wave][j][tq + 4 * i] = dots[j];
        __builtin_amdgcn_sched_barrier(0);   // one row at a time
      }
    }
    // this pass's V rows, in flight during the softmax
    u4 vr[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int vo = VB ? ((tq + 4 * i < n) ? ((pos0 + (p0 - i_lo) + tq + 4 * i) * D + col) * 2 : a.cap * D * 2)
                        : roff(i);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vp, vo, 0, 0);
    }
    __syncthreads();
    if (wave < NH && lane < PT) {  // online softmax update, wave j for head j
      const int j = wave;
      const float sv = lane < n ? ((W.sc[0][j][lane] + W.sc[1][j][lane]) + W.sc[2][j][lane]) + W.sc[3][j][lane]
                                : NEG_INF;
      const float mold = W.wm[j];
      float mx = sv;
#pragma unroll
      for (int o2 = 16; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
      const float mnew = fmaxf(mold, mx);
      const float p = (sv == NEG_INF) ? 0.0f : exp2f(sv - mnew);
      float l = p;
#pragma unroll
      for (int o2 = 16; o2 > 0; o2 >>= 1) l += __shfl_xor(l, o2);
      W.p[j][lane] = p;
      if (lane == 0) {
        const float alpha = (mold == NEG_INF) ? 0.0f : exp2f(mold - mnew);
        W.wa[j] = alpha;
        W.wm[j] = mnew;
        W.wl[j] = W.wl[j] * alpha + l;
      }
    }
    __syncthreads();
    {  // PV over this slice
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const float al = W.wa[j];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[j][k] *= al;
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const int tk = tq + 4 * i;
        float x[8];
        bf16x8(vr[i], x);
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float p = tk < n ? W.p[j][tk] : 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) o[j][k] = __builtin_fmaf(p, x[k], o[j][k]);
        }
        __builtin_amdgcn_sched_barrier(0);   // one row's conversions at a time
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < NH; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[j][k] += __shfl_xor(o[j][k], 16);
      o[j][k] += __shfl_xor(o[j][k], 32);
    }
  const int slot = a.win.slot0 + wblk;
  if (tq == 0)
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      if (j >= a.Gq) break;
      float* dst = a.partials + (((size_t)b * a.Hq + h * a.Gq + j) * a.pstride + slot) * (D + 2);
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[col + k] = o[j][k];
      if (wave == 0 && c == 0) {
        dst[D] = W.wm[j];
        dst[D + 1] = W.wl[j];
      }
    }
}

// INT2 streams of wave `wave`'s slice (quantization group) of one (sequence,
// kv head): K code chunks 2 wave and 2 wave + 1 of every 8 KiB tile, the
// group's scale|zero words, the slice's 2 KiB V code tile.
__device__ inline TileStreams wide_tile_streams(const DecodeArgs& a, int bh, int wave) {
  constexpr int D = 512;
  TileStreams s;
  s.kc = plane_rsrc(a.k.codes + kcode_byte(bh, a.cap, 0, 0, D), a.cap * 128);
  s.km = plane_rsrc(a.k.meta + meta_index(bh, a.cap, 0, wave, D), a.cap * 4);
  s.vm = plane_rsrc(a.v.meta + meta_index(bh, a.cap, 0, wave, D), a.cap * 4);
  s.vc = plane_rsrc(a.v.codes + (size_t)bh * (a.cap / kTile) * (4 * 2048), a.cap * 128);
  return s;
}

// Loads of tile t0 for one slice: lane_k = 2048 wave + 16 lane (K chunk
// 2 wave), lane_v = 2048 wave + 16 lane (V slice tile), lane_m = 16 blk.
__device__ inline TileRegs wide_load_tile(const TileStreams& s, int t0, int lane_c, int lane_m) {
  const int oc = t0 * 128, om = t0 * 4;
  TileRegs r;
  // in order of first use (loads return in issue order)
  r.k0 = __builtin_amdgcn_raw_buffer_load_b128(s.kc, lane_c, oc, kStreamOnce);
  r.k1 = __builtin_amdgcn_raw_buffer_load_b128(s.kc, lane_c + 1024, oc, kStreamOnce);
  r.km = __builtin_amdgcn_raw_buffer_load_b128(s.km, lane_m, om, 0);
  r.vm = __builtin_amdgcn_raw_buffer_load_b128(s.vm, lane_m, om, 0);
  __builtin_amdgcn_sched_barrier(0);
  r.v0 = __builtin_amdgcn_raw_buffer_load_b128(s.vc, lane_c, oc, kStreamOnce);
  r.v1 = __builtin_amdgcn_raw_buffer_load_b128(s.vc, lane_c + 1024, oc, kStreamOnce);
  __builtin_amdgcn_sched_barrier(0);
  return r;
}

// INT2 split with V kept bf16: QK^T as in the INT2 path (wave w = K group w,
// partial scores summed in shared memory), then the softmax weights of the
// tile go to the wave's own shared-memory row and PV runs in fp32 on the VALU
// over the tile's V rows (row-major, dims [128 w, 128 w + 128) of each):
// lane (tq, c) takes dims 8 c .. 8 c + 7 of rows tq + 4 i, i = 0..15, every
// load contiguous across 16 lanes; the tile's V rows are issued first and
// land during QK^T and the softmax.
template <int NH>
__device__ void wide_split_bf16v(const DecodeArgs& a, int bh, int b, int h, int split, WideSmem& W) {
  constexpr int D = 512;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int blk = lane >> 2, j = lane & 3;
  const int tq = lane >> 4, c = lane & 15;
  const int lo = a.plan.a0, hi = a.lens ? max(a.N, a.lens[b] - a.M) : a.plan.b0;   // this sequence's INT2 range
  const int tile_first = lo >> 6;
  const int ntiles = hi > lo ? ((hi - 1) >> 6) - tile_first + 1 : 0;
  const int S_ = a.plan.splits;
  auto split_start = [&](int s) -> int { return s >= S_ ? ntiles : s * ntiles / S_; };
  const int s_t0 = split_start(split);
  const int s_t1 = split_start(split + 1);
  const int t_last = max(s_t1 - 1, 0);
  const TileStreams st = wide_tile_streams(a, bh, wave);
  const __amdgpu_buffer_rsrc_t vfull = plane_rsrc(a.v.full + row_offset(bh, a.cap, 0, D), a.cap * D * 2);
  const int vnull = a.cap * D * 2;        // past the plane: loads zero
  const int lane_c = 2048 * wave + lane * 16, lane_m = blk * 16;
  const int col = 128 * wave + 8 * c;
  auto tile_t0 = [&](int ti) { return (tile_first + ti) << 6; };
  struct KRegs {
    u4 k0, k1, km;
  };
  // past the split's last tile the loads go through zero-length resources
  TileStreams none = st;
  none.kc = plane_rsrc(a.k.codes, 0);
  none.km = plane_rsrc(a.k.meta, 0);
  auto load_k = [&](int t0, bool live_tile = true) {
    const TileStreams& s = live_tile ? st : none;
    KRegs r;
    r.k0 = __builtin_amdgcn_raw_buffer_load_b128(s.kc, lane_c, t0 * 128, kStreamOnce);
    r.k1 = __builtin_amdgcn_raw_buffer_load_b128(s.kc, lane_c + 1024, t0 * 128, kStreamOnce);
    r.km = __builtin_amdgcn_raw_buffer_load_b128(s.km, lane_m, t0 * 4, 0);
    return r;
  };
  // q operands first (loads return in issue order: the first tile's work
  // then waits for q and that tile only)
  h4 qv[1][8];
  float qsum;
  int eq;
  const uint2* qlp[1] = {wide_q_operands(a, bh * 4 + wave, W.qlo[wave], qv[0], qsum, eq)};
  KRegs r[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k) r[k] = load_k(tile_t0(min(s_t0 + k, t_last)));
  __syncthreads();                        // W.qlo complete
  const float cK = ldexpf(1.0f, 24 - eq);
  const float zq = ldexpf(qsum, eq - 24);
  float m = NEG_INF, l = 0.0f;
  float o[NH][8];
#pragma unroll
  for (int jj = 0; jj < NH; ++jj)
#pragma unroll
    for (int k = 0; k < 8; ++k) o[jj][k] = 0.0f;

  int buf = 0;
  auto process = [&](const KRegs& cur, int t0) {
    // V rows of the tile (zero outside [lo, hi))
    u4 vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + tq + 4 * i;
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vfull, (t >= lo && t < hi) ? (t * D + col) * 2 : vnull, 0,
                                                    kStreamOnce);
    }
    f4 sa[1] = {{0, 0, 0, 0}};
    qk_word<1>(cur.k0.x, qv, qlp, 0, sa);
    qk_word<1>(cur.k0.y, qv, qlp, 1, sa);
    qk_word<1>(cur.k0.z, qv, qlp, 2, sa);
    qk_word<1>(cur.k0.w, qv, qlp, 3, sa);
    qk_word<1>(cur.k1.x, qv, qlp, 4, sa);
    qk_word<1>(cur.k1.y, qv, qlp, 5, sa);
    qk_word<1>(cur.k1.z, qv, qlp, 6, sa);
    qk_word<1>(cur.k1.w, qv, qlp, 7, sa);
    const uint32_t kmr[4] = {cur.km.x, cur.km.y, cur.km.z, cur.km.w};
    f4 part;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      part[rr] = cK * __builtin_fmaf(hi_half(kmr[rr]), zq, __builtin_fmaf(lo_half(kmr[rr]), sa[0][rr], 0.0f));
    W.u[buf][wave][lane] = part;
    __syncthreads();
    f4 u = ((W.u[buf][0][lane] + W.u[buf][1][lane]) + W.u[buf][2][lane]) + W.u[buf][3][lane];
    buf ^= 1;
    if (t0 < lo || t0 + 64 > hi) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = t0 + 4 * blk + rr;
        if (t < lo || t >= hi) u[rr] = NEG_INF;
      }
    }
    const float tmax = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
    if (__any(tmax > m)) {
      const float mnew = fmaxf(m, head_max(tmax));
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
      m = mnew;
#pragma unroll
      for (int jj = 0; jj < NH; ++jj) {
        const float al = lane_value(alpha, jj);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[jj][k] *= al;
      }
    }
    float p[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) p[rr] = __builtin_amdgcn_exp2f(u[rr] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    // weights to this wave's row of shared memory: head j, token 4 blk + rr
    *reinterpret_cast<f4*>(&W.pv[wave][j][4 * blk]) = f4{p[0], p[1], p[2], p[3]};
    wave_lds_sync();   // the wave's own writes are visible to its reads
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tk = tq + 4 * i;
      float x[8];
      bf16x8(vr[i], x);
#pragma unroll
      for (int jj = 0; jj < NH; ++jj) {
        const float pw = W.pv[wave][jj][tk];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[jj][k] = __builtin_fmaf(pw, x[k], o[jj][k]);
      }
      __builtin_amdgcn_sched_barrier(0);   // one row's conversions at a time
    }
  };

  // rounds of kDepth tiles with no exit in the middle (as in the INT2 splits)
  for (int ti = s_t0; ti < s_t1; ti += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int t = ti + k;
      if (t < s_t1) process(r[k], tile_t0(t));
      r[k] = load_k(tile_t0(min(t + kDepth, t_last)), t + kDepth < s_t1);
    }
  }

  const float lt = head_sum(l);
#pragma unroll
  for (int jj = 0; jj < NH; ++jj)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[jj][k] += __shfl_xor(o[jj][k], 16);
      o[jj][k] += __shfl_xor(o[jj][k], 32);
    }
  const int slot = a.plan.slot0 + split;
  if (tq == 0)
#pragma unroll
    for (int jj = 0; jj < NH; ++jj) {
      if (jj >= a.Gq) break;
      float* dst = a.partials + (((size_t)b * a.Hq + h * a.Gq + jj) * a.pstride + slot) * (D + 2);
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[col + k] = o[jj][k];
    }
  if (wave == 0 && lane < a.Gq) {
    float* dst = a.partials + (((size_t)b * a.Hq + h * a.Gq + lane) * a.pstride + slot) * (D + 2);
    dst[D] = m;
    dst[D + 1] = lt;
  }
}

// Grid: (sequence x kv head, plan.splits INT2 splits + win_blocks window
// blocks).  NH: query heads per kv head rounded up to 2 or 4 (the window
// blocks' register arrays; the matrix-core part always has 4 columns).  VB: V
// kept bf16 for every position (INT2 K only); each wave then holds a whole
// tile of V rows (64 registers, 16 KiB per wave in flight) and runs at 2 waves
// per SIMD.
template <int NH, bool VB>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(VB ? 2 : 4, VB ? 2 : 4)))
void decode_wide_kernel(DecodeArgs a) {
  constexpr int D = 512;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  __shared__ WideSmem W;
  const int y = (int)blockIdx.y;
  // window blocks first: their passes are latency-bound, so they start early
  // and run beside the INT2 streaming
  if (y < a.win_blocks) {
    wide_window_block<NH, VB>(a, bh, b, h, y, W);
    return;
  }
  const int split = y - a.win_blocks;
  if constexpr (VB) {
    wide_split_bf16v<NH>(a, bh, b, h, split, W);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int blk = lane >> 2, j = lane & 3;
  const int lo = a.plan.a0, hi = a.lens ? max(a.N, a.lens[b] - a.M) : a.plan.b0;   // this sequence's INT2 range
  const int tile_first = lo >> 6;
  const int ntiles = hi > lo ? ((hi - 1) >> 6) - tile_first + 1 : 0;
  auto split_start = [&](int s) -> int {
    const int S = a.plan.splits;
    return s >= S ? ntiles : s * ntiles / S;
  };
  const int s_t0 = split_start(split);
  const int s_t1 = split_start(split + 1);
  const int t_last = max(s_t1 - 1, 0);
  const TileStreams st = wide_tile_streams(a, bh, wave);
  const int lane_c = 2048 * wave + lane * 16, lane_m = blk * 16;
  auto tile_t0 = [&](int ti) { return (tile_first + ti) << 6; };
  // this slice's q operands (written by the rotation launch before this one)
  // and the V-scale maximum first: the first tile's work then waits for them
  // and that tile only (loads return in issue order)
  h4 qv[1][8];
  float qsum;
  int eq;
  const uint2* qlp[1] = {wide_q_operands(a, bh * 4 + wave, W.qlo[wave], qv[0], qsum, eq)};
  const float vmax = a.v.smax[bh];
  TileRegs r[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k) r[k] = wide_load_tile(st, tile_t0(min(s_t0 + k, t_last)), lane_c, lane_m);
  __syncthreads();                        // W.qlo complete
  const float cK = ldexpf(1.0f, 24 - eq);
  const float zq = ldexpf(qsum, eq - 24);
  int ev2 = 0;
  if (vmax > 0.0f) frexpf(vmax, &ev2);
  const int ev = (vmax > 0.0f) ? min(15 - ev2, 60) : 0;
  const int kA = ev - 4 * (blk & 1);
  const float kAf = (float)kA;
  const float cV = ldexpf(1.0f, 24 - ev);

  f4 o0[1] = {{0, 0, 0, 0}}, o1[1] = {{0, 0, 0, 0}};
  float m = NEG_INF, lA = 0.0f, lB = 0.0f, pzA = 0.0f, pzB = 0.0f;
  float cA = 0.0f, cB = 0.0f;

  // one 64-token tile: this slice's QK^T, the four slices' scores summed in
  // shared memory (fixed order, identical in every wave), the online softmax
  // (the same in every wave), this slice's PV
  auto process = [&](const TileRegs& cur, int t0, int buf) {
    f4 sa[1] = {{0, 0, 0, 0}};
    qk_word<1>(cur.k0.x, qv, qlp, 0, sa);
    qk_word<1>(cur.k0.y, qv, qlp, 1, sa);
    qk_word<1>(cur.k0.z, qv, qlp, 2, sa);
    qk_word<1>(cur.k0.w, qv, qlp, 3, sa);
    qk_word<1>(cur.k1.x, qv, qlp, 4, sa);
    qk_word<1>(cur.k1.y, qv, qlp, 5, sa);
    qk_word<1>(cur.k1.z, qv, qlp, 6, sa);
    qk_word<1>(cur.k1.w, qv, qlp, 7, sa);
    PHASE_FENCE();
    const uint32_t kmr[4] = {cur.km.x, cur.km.y, cur.km.z, cur.km.w};
    const uint32_t vmr[4] = {cur.vm.x, cur.vm.y, cur.vm.z, cur.vm.w};
    f4 part;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      part[r] = cK * __builtin_fmaf(hi_half(kmr[r]), zq, __builtin_fmaf(lo_half(kmr[r]), sa[0][r], 0.0f));
    W.u[buf][wave][lane] = part;
    __syncthreads();
    f4 u = ((W.u[buf][0][lane] + W.u[buf][1][lane]) + W.u[buf][2][lane]) + W.u[buf][3][lane];
    if (t0 < lo || t0 + 64 > hi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * blk + r;
        if (t < lo || t >= hi) u[r] = NEG_INF;
      }
    }
    const float tmax = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
    if (__any(tmax > m)) {
      const float mnew = fmaxf(m, head_max(tmax));
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lA *= alpha;
      lB *= alpha;
      pzA *= alpha;
      pzB *= alpha;
      const f4 al = {lane_value(alpha, 0), lane_value(alpha, 1), lane_value(alpha, 2), lane_value(alpha, 3)};
      o0[0] *= al;
      o1[0] *= al;
      m = mnew;
      cA = kAf - m;
      cB = cA - 2.0f;
    }
    float p[4];
    p[0] = __builtin_amdgcn_exp2f(u[0] + cA);
    p[1] = __builtin_amdgcn_exp2f(u[1] + cA);
    p[2] = __builtin_amdgcn_exp2f(u[2] + cB);
    p[3] = __builtin_amdgcn_exp2f(u[3] + cB);
    lA += p[0] + p[1];
    lB += p[2] + p[3];
    pzA = __builtin_fmaf(p[0], hi_half(vmr[0]), __builtin_fmaf(p[1], hi_half(vmr[1]), pzA));
    pzB = __builtin_fmaf(p[2], hi_half(vmr[2]), __builtin_fmaf(p[3], hi_half(vmr[3]), pzB));
    h4 pv1[1], pl1[1];
    pv_operands(vmr, p, pv1[0], pl1[0]);
    PHASE_FENCE();
    pv_word<1, 0>(cur.v0.x, pv1, pl1, o0, o1);
    pv_word<1, 1>(cur.v0.y, pv1, pl1, o0, o1);
    pv_word<1, 2>(cur.v0.z, pv1, pl1, o0, o1);
    pv_word<1, 3>(cur.v0.w, pv1, pl1, o0, o1);
    pv_word<1, 4>(cur.v1.x, pv1, pl1, o0, o1);
    pv_word<1, 5>(cur.v1.y, pv1, pl1, o0, o1);
    pv_word<1, 6>(cur.v1.z, pv1, pl1, o0, o1);
    pv_word<1, 7>(cur.v1.w, pv1, pl1, o0, o1);
  };

  // Rounds of kDepth tiles with no exit in the middle (a missing tile is
  // skipped, its reload still issued, through zero-length resources past the
  // split's last tile): every path reaches the loop head with the same loads
  // in flight in the same order, so a tile's work waits for its own loads
  // only (with an exit after each tile the loop head waited for every load)
  TileStreams none = st;
  none.kc = plane_rsrc(a.k.codes, 0);
  none.km = plane_rsrc(a.k.meta, 0);
  none.vm = plane_rsrc(a.v.meta, 0);
  none.vc = plane_rsrc(a.v.codes, 0);
  int buf = 0;
  for (int ti = s_t0; ti < s_t1; ti += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int t = ti + k;
      if (t < s_t1) {
        process(r[k], tile_t0(t), buf);
        buf ^= 1;
      }
      r[k] = wide_load_tile(t + kDepth < s_t1 ? st : none, tile_t0(min(t + kDepth, t_last)), lane_c, lane_m);
    }
  }

  const float l = head_sum(ldexpf(__builtin_fmaf(4.0f, lB, lA), -kA));
  const float pz = head_sum(ldexpf(__builtin_fmaf(4.0f, pzB, pzA), -kA));
  const float pzr[4] = {lane_value(pz, 0), lane_value(pz, 1), lane_value(pz, 2), lane_value(pz, 3)};
  const int slot = a.plan.slot0 + split;
#pragma unroll
  for (int r2 = 0; r2 < 4; ++r2) {
    if (r2 >= a.Gq) break;
    float* dst = a.partials + (((size_t)b * a.Hq + h * a.Gq + r2) * a.pstride + slot) * (D + 2);
    dst[128 * wave + 4 * blk + j] = __builtin_fmaf(o0[0][r2], cV, pzr[r2]);
    dst[128 * wave + 64 + 4 * blk + j] = __builtin_fmaf(o1[0][r2], cV, pzr[r2]);
    if (wave == 0 && lane == r2) {
      dst[D] = m;
      dst[D + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_qrot(const QRotArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hkv));
  if (a.D == 128)
    hipLaunchKernelGGL(qrot_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(qrot_kernel<512>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeArgs& a, int B, hipStream_t s) {
  dim3 grid((unsigned)(B * a.Hkv), (unsigned)a.plan.splits);
  if (a.D == 128)
    hipLaunchKernelGGL(decode_valu_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_valu_kernel<512>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

int decode_mfma_resident_blocks(int device, int G) {
  int per_cu = 0, cus = 0;
  const hipError_t e =
      G == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_kernel<4, 2, false, false>, 256, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_kernel<4, 1, false, false>, 256, 0);
  if (e != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) cus = 1;
  return per_cu * cus;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int waves_per_block, hipStream_t s) {
  (void)waves_per_block;   // the fused window blocks need 4 waves
  dim3 grid((unsigned)(B * a.Hkv), (unsigned)(a.one_round ? a.plan.splits : a.plan.splits + a.win_blocks));
  auto launch = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, a); };
  if (a.G == 2) {
    if (a.one_round) launch(decode_mfma_kernel<4, 2, true, false>);
    else if (a.self_rotate) launch(decode_mfma_kernel<4, 2, false, true>);
    else launch(decode_mfma_kernel<4, 2, false, false>);
  } else {
    if (a.one_round) launch(decode_mfma_kernel<4, 1, true, false>);
    else if (a.self_rotate) launch(decode_mfma_kernel<4, 1, false, true>);
    else launch(decode_mfma_kernel<4, 1, false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_decode_prologue(const DecodeArgs& a, int B, hipStream_t s) {
  dim3 grid((unsigned)(B * a.Hkv), (unsigned)(a.G + a.app_blocks));
  if (a.G == 2)
    hipLaunchKernelGGL((decode_prologue_kernel<2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_prologue_kernel<1>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_wide_qrot(const DecodeArgs& a, int B, hipStream_t s) {
  if (a.app_blocks > 0)
    hipLaunchKernelGGL(wide_prologue_kernel, dim3((unsigned)(B * a.Hkv), 4 + 8), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(wide_qrot_kernel, dim3((unsigned)(B * a.Hkv), 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_wide(const DecodeArgs& a, int B, hipStream_t s) {
  dim3 grid((unsigned)(B * a.Hkv), (unsigned)(a.plan.splits + a.win_blocks));
  const bool vb = a.v.is_bf16 != 0;
  if (a.Gq <= 2) {
    if (vb)
      hipLaunchKernelGGL((decode_wide_kernel<2, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_wide_kernel<2, false>), grid, dim3(256), 0, s, a);
  } else {
    if (vb)
      hipLaunchKernelGGL((decode_wide_kernel<4, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_wide_kernel<4, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.D == 128)
    hipLaunchKernelGGL((combine_kernel<128, 1, kMaxGq>), dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_wide_kernel, dim3((unsigned)(a.B * a.Hkv), 4, (unsigned)(a.Hq / a.Hkv)),
                       dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
