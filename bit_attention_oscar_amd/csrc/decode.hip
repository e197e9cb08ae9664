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
//   qrot_kernel         q_rot = q @ R_K * scale * log2(e) (fp32), per-group sums,
//                       and the fp16 operand registers of the matrix-core kernel
//   decode_valu_kernel  general split-K kernel: any head_dim / GQA / dtype,
//                       per-token precision chosen by position
//   decode_mfma_kernel  INT2 range, head_dim 128, 4 query heads per kv head:
//                       4x4x4 f16 matrix-core QK^T and PV on raw codes
//   combine_kernel      log-sum-exp merge of the splits and o = o' @ R_V^T
#include <math.h>
#include "common.h"

namespace oscar {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

#define NEG_INF (-__builtin_inff())

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

template <int D>
__global__ __launch_bounds__(128) void qrot_kernel(QRotArgs a) {
  constexpr int PER = D / 128;
  const int tid = threadIdx.x;
  const int bq = blockIdx.x;                 // b * Hq + head
  __shared__ float xs[D];
  __shared__ float vs[D];
  __shared__ float red[4][4];
  for (int d = tid; d < D; d += 128) xs[d] = bf16_to_f32(a.q[(size_t)bq * D + d]);
  __syncthreads();
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  for (int e = 0; e < D; ++e) {
    const float x = xs[e];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(x, a.rk[(size_t)e * D + tid + 128 * i], acc[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float v = acc[i] * a.scale_log2;
    vs[tid + 128 * i] = v;
    a.qrot[(size_t)bq * D + tid + 128 * i] = v;
    amax = fmaxf(amax, fabsf(v));
  }
  // per-group sums (group g = dims [128 g, 128 g + 128) = element g of every thread)
  const int wave = tid >> 6, lane = tid & 63;
  float gs[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < PER; ++i) gs[i] = wsum(acc[i] * a.scale_log2);
  amax = wmax(amax);
  if (lane == 0) {
    for (int g = 0; g < 4; ++g) red[wave][g] = gs[g];
    red[2 + wave][0] = amax;
  }
  __syncthreads();
  const float gmax = fmaxf(red[2][0], red[3][0]);
  int e2 = 0;
  if (gmax > 0.0f) frexpf(gmax, &e2);
  const int eq = (gmax > 0.0f) ? 15 - e2 : 0;          // |q| * 2^eq < 2^15
  if (tid < 8) {
    float v = 0.0f;
    if (tid < PER) v = red[0][tid] + red[1][tid];
    if (tid == 4) v = ldexpf(1.0f, 24 - eq);           // cK: undoes 2^eq and the 2^-24 code scale
    a.qaux[(size_t)bq * 8 + tid] = v;
  }
  if (a.want_swz && D == 128) {
    // fp16 operand registers: [b*Hkv + kvh][lane 64][w 8][k 4], lane = 4*blk + j
    // holds query head j of the kv head; all four blocks of a lane group pp
    // hold the same chunk (w, pp), broadcast by the instruction.
    const int Gq = a.Hq / a.Hkv;
    const int b = bq / a.Hq, head = bq - b * a.Hq;
    const int kvh = head / Gq, j = head - kvh * Gq;
    uint16_t* dst = a.qswz + ((size_t)(b * a.Hkv + kvh) * 64) * 32;
    for (int e = tid; e < 16 * 32; e += 128) {
      const int m = e >> 5, w = (e >> 2) & 7, k = e & 3;
      const int lane_id = 4 * m + j;
      const int pp = lane_id >> 4;
      const int d = qk_dim(w, pp, k);
      const float v = ldexpf(vs[d], eq - 2 * (d & 3));
      dst[(size_t)lane_id * 32 + w * 4 + k] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
  }
}

// ---------------------------------------------------------------------------
// general VALU split-K kernel
// ---------------------------------------------------------------------------

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
  const uint32_t meta = P.meta[meta_offset(bh, cap, t, D) + d0 / kGroup];
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta >> 16));
  if (!P.tiled) {
    const uint8_t* row = P.codes + kcode_offset(bh, cap, t, D);
    for (int i = 0; i < n; i += 16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(row + (d0 + i) / 4);
#pragma unroll
      for (int k = 0; k < 16; ++k) out[i + k] = __builtin_fmaf(s, (float)((w >> (2 * k)) & 3u), z);
    }
  } else {
    for (int i = 0; i < n; ++i) {
      int bit;
      const size_t off = vcode_byte(bh, cap, t, d0 + i, D, &bit);
      out[i] = __builtin_fmaf(s, (float)((P.codes[off] >> bit) & 3u), z);
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
  const uint32_t meta = P.meta[meta_offset(bh, cap, t, D) + d / kGroup];
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta >> 16));
  uint32_t c;
  if (!P.tiled) {
    c = (P.codes[kcode_offset(bh, cap, t, D) + d / 4] >> (2 * (d & 3))) & 3u;
  } else {
    int bit;
    const size_t off = vcode_byte(bh, cap, t, d, D, &bit);
    c = (P.codes[off] >> bit) & 3u;
  }
  return __builtin_fmaf(s, (float)c, z);
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

  const int len = (a.plan.b0 - a.plan.a0) + (a.plan.b1 - a.plan.a1);
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
          load_row_values<D>(a.k, bh, t, a.T, a.N, a.M, a.cap, part * PART + c0, 16, kv);
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
          const float vv = load_value<D>(a.v, bh, t, a.T, a.N, a.M, a.cap, d);
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
    float* dst = a.partials + (((size_t)b * a.Hq + h * Gq + hq) * kMaxSplits + slot) * (D + 2);
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

template <int W>
__device__ inline void qk_word(uint32_t word, h4 q, f4& sa, f4& sb) {
  uint32_t c[8];
  split_codes(word, c);
  sa = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[0], c[1]), q, sa, 0, 0, 4);
  sb = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[2], c[3]), q, sb, 0, 0, 5);
  sa = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[4], c[5]), q, sa, 0, 0, 6);
  sb = __builtin_amdgcn_mfma_f32_4x4x4f16(as_h4(c[6], c[7]), q, sb, 0, 0, 7);
}

template <int W>
__device__ inline void pv_word(uint32_t word, h4 p, f4& o0, f4& o1) {
  uint32_t c[8];
  split_codes(word, c);
  // word W holds tokens 8W..8W+7 = blocks beta 2W (pairs 0,1) and 2W+1 (pairs 2,3);
  // positions 0-3 are the low half of head_dim, 4-7 the high half
  o0 = __builtin_amdgcn_mfma_f32_4x4x4f16(p, as_h4(c[0], c[1]), o0, 4, 2 * W, 0);
  o1 = __builtin_amdgcn_mfma_f32_4x4x4f16(p, as_h4(c[4], c[5]), o1, 4, 2 * W, 0);
  o0 = __builtin_amdgcn_mfma_f32_4x4x4f16(p, as_h4(c[2], c[3]), o0, 4, 2 * W + 1, 0);
  o1 = __builtin_amdgcn_mfma_f32_4x4x4f16(p, as_h4(c[6], c[7]), o1, 4, 2 * W + 1, 0);
}

template <int WPB>
__global__ __launch_bounds__(64 * WPB) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int blk = lane >> 2, j = lane & 3;
  const int lo = a.plan.a0, hi = a.plan.b0;       // INT2 token range
  const int tile_first = lo >> 6;
  const int ntiles = ((hi - 1) >> 6) - tile_first + 1;
  const int tps = a.plan.chunk >> 6;
  const int s_t0 = (int)blockIdx.y * tps;
  const int s_t1 = min(s_t0 + tps, ntiles);

  // q operands: 8 words x 4 fp16
  const uint4* qp = reinterpret_cast<const uint4*>(a.qswz + ((size_t)bh * 64 + lane) * 32);
  const uint4 q01 = qp[0], q23 = qp[1], q45 = qp[2], q67 = qp[3];
  const h4 qv[8] = {as_h4(q01.x, q01.y), as_h4(q01.z, q01.w), as_h4(q23.x, q23.y), as_h4(q23.z, q23.w),
                    as_h4(q45.x, q45.y), as_h4(q45.z, q45.w), as_h4(q67.x, q67.y), as_h4(q67.z, q67.w)};
  const float* aux = a.qaux + ((size_t)b * a.Hq + h * 4 + j) * 8;
  const float cK = aux[4];
  const float zq = aux[0] / cK;                    // sum(q_rot) in units of the raw dot
  const float vmax = a.v.smax[bh];
  int ev2 = 0;
  if (vmax > 0.0f) frexpf(vmax, &ev2);
  const int ev = (vmax > 0.0f) ? 15 - ev2 : 0;     // s_V * 2^ev < 2^15
  const float fvA = ldexpf(1.0f, ev - 4 * (blk & 1));
  const float fvB = ldexpf(1.0f, ev - 4 * (blk & 1) - 2);
  const float cV = ldexpf(1.0f, 24 - ev);

  f4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
  float m = NEG_INF, l = 0.0f, pz = 0.0f;
  const size_t vtile_base = (size_t)bh * (a.cap / kTile);

  for (int ti = s_t0 + wave; ti < s_t1; ti += WPB) {
    const int t0 = (tile_first + ti) << 6;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k.codes + kcode_offset(bh, a.cap, t0 + lane, D));
    const uint4 k0 = kp[0], k1 = kp[1];
    const uint4 km = *reinterpret_cast<const uint4*>(a.k.meta + meta_offset(bh, a.cap, t0 + 4 * blk, D));
    const uint4 vm = *reinterpret_cast<const uint4*>(a.v.meta + meta_offset(bh, a.cap, t0 + 4 * blk, D));
    const uint4* vp = reinterpret_cast<const uint4*>(a.v.codes + (vtile_base + (t0 >> 6)) * 2048 + lane * 32);
    const uint4 v0 = vp[0], v1 = vp[1];

    f4 sa = {0, 0, 0, 0}, sb = {0, 0, 0, 0};
    qk_word<0>(k0.x, qv[0], sa, sb);
    qk_word<1>(k0.y, qv[1], sa, sb);
    qk_word<2>(k0.z, qv[2], sa, sb);
    qk_word<3>(k0.w, qv[3], sa, sb);
    qk_word<4>(k1.x, qv[4], sa, sb);
    qk_word<5>(k1.y, qv[5], sa, sb);
    qk_word<6>(k1.z, qv[6], sa, sb);
    qk_word<7>(k1.w, qv[7], sa, sb);
    const f4 sc = sa + sb;

    const uint32_t kmr[4] = {km.x, km.y, km.z, km.w};
    const uint32_t vmr[4] = {vm.x, vm.y, vm.z, vm.w};
    float u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = __builtin_fmaf(lo_half(kmr[r]), sc[r], hi_half(kmr[r]) * zq);
    if (t0 < lo || t0 + 64 > hi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * blk + r;
        if (t < lo || t >= hi) u[r] = NEG_INF;
      }
    }
    float mt = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 4));
    mt = fmaxf(mt, __shfl_xor(mt, 8));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, cK * mt);
    const float alpha = exp2f(m - mnew);
    m = mnew;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = exp2f(__builtin_fmaf(cK, u[r], -mnew));
    l = __builtin_fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    float pzt = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) pzt = __builtin_fmaf(p[r], hi_half(vmr[r]), pzt);
    pz = __builtin_fmaf(pz, alpha, pzt);
    const h4 pv = {(_Float16)(p[0] * lo_half(vmr[0]) * fvA), (_Float16)(p[1] * lo_half(vmr[1]) * fvA),
                   (_Float16)(p[2] * lo_half(vmr[2]) * fvB), (_Float16)(p[3] * lo_half(vmr[3]) * fvB)};
    const f4 al = {__shfl(alpha, 0), __shfl(alpha, 1), __shfl(alpha, 2), __shfl(alpha, 3)};
    o0 *= al;
    o1 *= al;
    pv_word<0>(v0.x, pv, o0, o1);
    pv_word<1>(v0.y, pv, o0, o1);
    pv_word<2>(v0.z, pv, o0, o1);
    pv_word<3>(v0.w, pv, o0, o1);
    pv_word<4>(v1.x, pv, o0, o1);
    pv_word<5>(v1.y, pv, o0, o1);
    pv_word<6>(v1.z, pv, o0, o1);
    pv_word<7>(v1.w, pv, o0, o1);
  }

  // per-head totals of l and sum(p z_V) over the 16 lanes of each head
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) {
    l += __shfl_xor(l, o);
    pz += __shfl_xor(pz, o);
  }
  __shared__ float sm[WPB][4], sl[WPB][4];
  __shared__ float so[WPB][4][D];
  if (lane < 4) {
    sm[wave][lane] = m;
    sl[wave][lane] = l;
  }
  const float pzr[4] = {__shfl(pz, 0), __shfl(pz, 1), __shfl(pz, 2), __shfl(pz, 3)};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    so[wave][r][4 * blk + j] = __builtin_fmaf(o0[r], cV, pzr[r]);
    so[wave][r][64 + 4 * blk + j] = __builtin_fmaf(o1[r], cV, pzr[r]);
  }
  __syncthreads();
  const int slot = a.plan.slot0 + (int)blockIdx.y;
  for (int idx = threadIdx.x; idx < 4 * D; idx += 64 * WPB) {
    const int r = idx / D, d = idx - r * D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < WPB; ++w) M = fmaxf(M, sm[w][r]);
    float O = 0.0f, L = 0.0f;
    if (M != NEG_INF) {
#pragma unroll
      for (int w = 0; w < WPB; ++w) {
        const float sw = exp2f(sm[w][r] - M);
        O = __builtin_fmaf(so[w][r][d], sw, O);
        L = __builtin_fmaf(sl[w][r], sw, L);
      }
    }
    float* dst = a.partials + (((size_t)b * a.Hq + h * 4 + r) * kMaxSplits + slot) * (D + 2);
    dst[d] = O;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// combine + V un-rotation
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  constexpr int PER = D / 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t row = blockIdx.x;                       // b * Hq + head
  const float* P = a.partials + row * kMaxSplits * (D + 2);
  __shared__ float wsl[kMaxSplits];
  __shared__ float os[D];
  __shared__ float red[2];
  float mx = NEG_INF;
  for (int s = tid; s < a.nslots; s += 128) mx = fmaxf(mx, P[(size_t)s * (D + 2) + D]);
  mx = wmax(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  __syncthreads();
  float L = 0.0f;
  for (int s = tid; s < a.nslots; s += 128) {
    const float ms = P[(size_t)s * (D + 2) + D];
    const float w = (ms == NEG_INF) ? 0.0f : exp2f(ms - M);
    wsl[s] = w;
    L = __builtin_fmaf(P[(size_t)s * (D + 2) + D + 1], w, L);
  }
  L = wsum(L);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  const float inv = 1.0f / (red[0] + red[1]);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = tid + 128 * i;
    float acc = 0.0f;
    for (int s = 0; s < a.nslots; ++s) acc = __builtin_fmaf(P[(size_t)s * (D + 2) + d], wsl[s], acc);
    os[d] = acc * inv;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = tid + 128 * i;
    float acc = 0.0f;
    for (int e = 0; e < D; ++e) acc = __builtin_fmaf(os[e], a.rvT[(size_t)e * D + d], acc);
    const size_t o = row * D + d;
    if (a.out_dtype == 0)
      reinterpret_cast<float*>(a.out)[o] = acc;
    else if (a.out_dtype == 1)
      reinterpret_cast<uint16_t*>(a.out)[o] = f32_to_bf16(acc);
    else
      reinterpret_cast<uint16_t*>(a.out)[o] = __builtin_bit_cast(uint16_t, (_Float16)acc);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_qrot(const QRotArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hq));
  if (a.D == 128)
    hipLaunchKernelGGL(qrot_kernel<128>, grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(qrot_kernel<512>, grid, dim3(128), 0, s, a);
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

hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int waves_per_block, hipStream_t s) {
  dim3 grid((unsigned)(B * a.Hkv), (unsigned)a.plan.splits);
  switch (waves_per_block) {
    case 1: hipLaunchKernelGGL(decode_mfma_kernel<1>, grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(decode_mfma_kernel<2>, grid, dim3(128), 0, s, a); break;
    case 8: hipLaunchKernelGGL(decode_mfma_kernel<8>, grid, dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.B * a.Hq));
  if (a.D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<512>, grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
