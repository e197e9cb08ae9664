// Chunked-prefill attention over the mixed INT2 + bf16 cache (head_dim 128 and 512).
//
// The serving hosts run a prefill backend beside the decode one (RotationZoo
// "How to use", the sglang launch's attention backends).  Here the queries of
// the last n cached positions T - n .. T - 1 attend causally over the cache as
// it stands after their chunk was appended: query i, at position p = T - n + i,
// reads positions [0, p]; the sink and recent windows of the current length T
// give their bf16 values, every other position its INT2 codes with the
// per-group fp16 scale and zero ("OSCAR: 2-bit KV Cache Quantization for
// SGLang and llama.cpp", "What OSCAR compresses").  q is rotated by R_K and the
// output un-rotated by R_V^T, as in the decode step.
//
// Block = 4 waves, one (sequence, kv head) and 64 query rows (64 / Gq queries
// x Gq heads of the kv head; wave w owns rows [16 w, 16 w + 16)).  Per 64-token
// key tile:
//   - the block stages the K tile [token][dim] and the V tile transposed
//     [dim][token] in shared memory as bf16 operands: INT2 positions as their
//     codes (0..3, exact in bf16) with the token's scale and zero kept aside,
//     window positions as their bf16 values (scale 1, zero 0);
//   - S = q K^T on v_mfma_f32_16x16x32_bf16, with q split into two bf16 pieces
//     (hi = bf16(q), lo = bf16(q - hi)) so that q keeps 16 significant bits;
//     the score of an INT2 token is s_K (q . c) + z_K (sum of q), in log2 units
//     (q carries softmax scale x log2 e);
//   - causal mask, online softmax per row;
//   - O += (p s_V) V on the matrix cores, p s_V split into two bf16 pieces the
//     same way; the zero's share (sum of p z_V per row) is added at the end.
// Last, o' = O / l, and o = o' R_V^T (or o' itself when the V rotation is
// absorbed).
#include "append_impl.h"
#include "prefill_attn.h"

#include <type_traits>

namespace oscar {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

struct alignas(16) PASmem {
  union {
    float rows[64][132];           // q rows before the rotation; o' rows before the un-rotation
    struct {
      uint16_t kt[64][136];        // K operand tile [token][dim], bf16 bits
      uint16_t vt[128][72];        // V operand tile [dim][token], bf16 bits
      float pf[64][68];            // p s_V [row][token], split into bf16 pieces when read
    } t;
  };
  float ks[64], kz[64], vs[64], vz[64];   // per-token scale and zero of the tile
  float qsum[64];                         // per row: sum of q over dims (both pieces)
};

// Two codes as bf16 operands in one word: x holds code c0 in bits 0-1 and c1
// in bits 16-17; the result is bf16(c0) | bf16(c1) << 16, through a byte
// permutation of a table of the bf16 bytes of 0, 1, 2, 3 (low bytes 00 80 00
// 40, high bytes 00 3F 40 40): selector byte i picks table byte c or 4 + c.
__device__ inline uint32_t codes2_bf16(uint32_t x) {
  const uint32_t sel = x * 0x0101u + 0x04000400u;
  return __builtin_amdgcn_perm(0x40403F00u, 0x40008000u, sel);
}

// bf16 operand words of the 8 codes at bits 2k of a 16-bit chunk w (values in
// order: word e holds codes 2e and 2e + 1)
__device__ inline u32x4_t codes8_bf16(uint32_t w) {
  const uint32_t v = (w & 0xFFFFu) | (((w & 0xFFFFu) >> 2) << 16);   // code 2e at bit 4e, code 2e+1 at bit 4e + 16
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = codes2_bf16((v >> (4 * e)) & 0x00030003u);
  return o;
}

// x = hi + lo to 16 significant bits: hi = bf16(x), lo = bf16(x - hi), both
// round to nearest even (the hardware conversion)
__device__ inline void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = __builtin_bit_cast(uint16_t, (__bf16)x);
  lo = __builtin_bit_cast(uint16_t, (__bf16)(x - bf16_to_f32(hi)));
}

__device__ inline void store_prefill_out(const PrefillAttnArgs& a, size_t o, float v) {
  if (a.out_dtype == 0)
    reinterpret_cast<float*>(a.out)[o] = v;
  else if (a.out_dtype == 1)
    reinterpret_cast<uint16_t*>(a.out)[o] = f32_to_bf16(v);
  else
    reinterpret_cast<uint16_t*>(a.out)[o] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// row r of the block -> query index (clamped to the last query) and query head
__device__ inline int row_query(const PrefillAttnArgs& a, int i0, int r) { return min(i0 + r / a.Gq, a.n - 1); }

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int D = 128;
  __shared__ PASmem S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const int QB = 64 / a.Gq;                       // queries per block
  const int i0 = (int)blockIdx.y * QB;
  const int T = a.lens ? a.lens[b] : a.T;          // this sequence's tokens (ragged batch: its own)
  const int sink_end = min(a.N, T), rec_begin = max(a.N, T - a.M);

  // ---- q rows (bf16 -> fp32), rotation by R_K, scale x log2 e
  for (int idx = tid; idx < 64 * D; idx += 256) {
    const int r = idx >> 7, d = idx & 127;
    const int i = row_query(a, i0, r), hq = h * a.Gq + r % a.Gq;
    S.rows[r][d] = bf16_to_f32(a.q[(((size_t)b * a.n + i) * a.Hq + hq) * D + d]);
  }
  __syncthreads();
  {
    const int d = tid & 127, r0 = tid >> 7;       // rows r0, r0 + 2, ..., 32 of them
    float acc[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = 0.0f;
    for (int e = 0; e < D; ++e) {
      const float re = a.rk[e * D + d];
#pragma unroll
      for (int k = 0; k < 32; ++k) acc[k] = __builtin_fmaf(S.rows[r0 + 2 * k][e], re, acc[k]);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32; ++k) S.rows[r0 + 2 * k][d] = acc[k] * a.scale_log2;
  }
  __syncthreads();
  // A operands: lane (m, kq) holds row 16 wave + m, dims 32 ks + kq .. + 8
  const int m = lane & 15, kq = 8 * (lane >> 4);
  u32x4_t qh[4], ql[4];
  float qpart = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t h0, l0, h1, l1;
      split_bf16(S.rows[16 * wave + m][32 * ks + kq + 2 * e], h0, l0);
      split_bf16(S.rows[16 * wave + m][32 * ks + kq + 2 * e + 1], h1, l1);
      qh[ks][e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      ql[ks][e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      qpart += (bf16_to_f32(h0) + bf16_to_f32(l0)) + (bf16_to_f32(h1) + bf16_to_f32(l1));
    }
  }
  qpart += __shfl_xor(qpart, 16);
  qpart += __shfl_xor(qpart, 32);
  if (lane < 16) S.qsum[16 * wave + m] = qpart;
  // (read back below by other lanes of the same wave, after an LDS wait and a
  // wave barrier)

  // ---- key tiles
  // accumulator layout (S and O): register i of a 16 x 16 block is row
  // 16 wave + 4 (lane >> 4) + i, column 16 cb + (lane & 15)
  int prow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) prow[i] = T - a.n + row_query(a, i0, 16 * wave + 4 * (lane >> 4) + i);
  const int p_max = T - a.n + min(i0 + QB - 1, a.n - 1);
  const int ntiles = (p_max >> 6) + 1;
  // a tile whose last token is at or before the block's first query position
  // needs no causal mask: every score in it is finite
  const int p_min = T - a.n + i0;
  // per-row q sums in registers (rows of this wave, written by this wave)
  wave_lds_sync();
  float qs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qs[i] = S.qsum[16 * wave + 4 * (lane >> 4) + i];
  float mrun[4], lrun[4], zrun[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrun[i] = kNegInf;
    lrun[i] = 0.0f;
    zrun[i] = 0.0f;
  }
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0, 0, 0, 0};

  const PlaneDev& K = a.k;
  const PlaneDev& V = a.v;
  auto half_f32 = [](uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); };
  for (int tt = 0; tt < ntiles; ++tt) {
    const int t0 = tt << 6;
    __syncthreads();                              // the previous tile's operands are consumed
    if (tid < 128) {
      // V codes: thread (record l = tid % 64, dim half dh = tid / 64) writes dim
      // ds = l + 64 dh of all 64 tokens.  The 2 KiB tile holds 64 lane records
      // of 32 bytes in two 1 KiB halves; record byte rec (= 2 k + dh for
      // dim ds) carries tokens 8 (k / 2) + (k % 2) + {0, 2, 4, 6} at bits
      // {0, 2, 4, 6}: bytes k = 2G and 2G + 1 give tokens 8G .. 8G + 7.
      const int l = tid & 63, dh = tid >> 6, ds = l + 64 * dh;
      if (!V.is_bf16) {
        const uint8_t* vt = V.codes + vcode_tile_base(bh, a.cap, t0, 0, D);
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(vt + 16 * l);          // rec 0..15
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(vt + 1024 + 16 * l);   // rec 16..31
#pragma unroll
        for (int G = 0; G < 8; ++G) {
          const int re = 4 * G + dh, ro = 4 * G + 2 + dh;            // record bytes of the even / odd tokens
          const u32x4_t& c = G < 4 ? c0 : c1;
          const uint32_t be = (c[(re & 15) >> 2] >> (8 * (re & 3))) & 0xFFu;
          const uint32_t bo = (c[(ro & 15) >> 2] >> (8 * (ro & 3))) & 0xFFu;
          const uint32_t v = be | (bo << 16);                        // token 8G + 2e at bit 2e, 8G + 2e + 1 at 16 + 2e
          u32x4_t o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = codes2_bf16((v >> (2 * e)) & 0x00030003u);
          *reinterpret_cast<u32x4_t*>(&S.t.vt[ds][8 * G]) = o;
        }
      }
      if (tid < 64) {
        const int t = t0 + tid;
        float sv = 0.0f, zv = 0.0f;
        if (t < T) {
          if (V.is_bf16 || t < sink_end || t >= rec_begin) {
            sv = 1.0f;
          } else {
            const uint32_t mw = V.meta[meta_index(bh, a.cap, t, 0, D)];
            sv = half_f32(mw & 0xFFFFu);
            zv = half_f32(mw >> 16);
          }
        }
        S.vs[tid] = sv;
        S.vz[tid] = zv;
      }
    } else {
      // K: thread (token tk = (tid - 128) / 2, dim half kh) writes dims
      // [64 kh, 64 kh + 64) of token tk: 16 code bytes, or the bf16 row piece
      const int tk = (tid - 128) >> 1, kh = tid & 1, t = t0 + tk;
      uint16_t* dst = &S.t.kt[tk][64 * kh];
      float sk = 0.0f, zk = 0.0f;
      if (t >= T) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(dst + 8 * i) = u32x4_t{0, 0, 0, 0};
      } else if (K.is_bf16 || t < sink_end || t >= rec_begin) {
        const uint16_t* src = K.is_bf16 ? K.full + row_offset(bh, a.cap, t, D)
                            : t < sink_end ? K.sink + row_offset(bh, a.N, t, D)
                                           : K.ring + row_offset(bh, a.M, t % a.M, D);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4_t*>(dst + 8 * i) = *reinterpret_cast<const u32x4_t*>(src + 64 * kh + 8 * i);
        sk = 1.0f;
      } else {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(K.codes + kcode_byte(bh, a.cap, t, 16 * kh, D));
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(dst + 8 * i) = codes8_bf16(w[i >> 1] >> (16 * (i & 1)));
        const uint32_t mw = K.meta[meta_index(bh, a.cap, t, 0, D)];
        sk = half_f32(mw & 0xFFFFu);
        zk = half_f32(mw >> 16);
      }
      if (kh == 0) {
        S.ks[tk] = sk;
        S.kz[tk] = zk;
      }
    }
    const bool tile_has_window = V.is_bf16 || t0 < sink_end || t0 + 64 > rec_begin || t0 + 64 > T;   // block-uniform
    if (tile_has_window) {
      // V rows of window tokens (every token of a bf16 plane) overwrite their
      // columns; positions past T are zeroed.  Thread: token tid / 4, dims
      // [32 (tid % 4), + 32).
      __syncthreads();                            // the code pass has written every column
      const int tk = tid >> 2, qd = tid & 3, t = t0 + tk;
      if (t >= T) {
#pragma unroll
        for (int e = 0; e < 32; ++e) S.t.vt[32 * qd + e][tk] = 0;
      } else if (V.is_bf16 || t < sink_end || t >= rec_begin) {
        const uint16_t* src = V.is_bf16 ? V.full + row_offset(bh, a.cap, t, D)
                            : t < sink_end ? V.sink + row_offset(bh, a.N, t, D)
                                           : V.ring + row_offset(bh, a.M, t % a.M, D);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + 32 * qd + 8 * i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S.t.vt[32 * qd + 8 * i + 2 * e][tk] = (uint16_t)(w[e] & 0xFFFFu);
            S.t.vt[32 * qd + 8 * i + 2 * e + 1][tk] = (uint16_t)(w[e] >> 16);
          }
        }
      }
    }
    __syncthreads();

    // S = q K^T for the wave's 16 rows and the tile's 64 tokens.  A wave
    // issuing matrix-core work runs at raised priority, so the other block's
    // waves fill the gaps with their softmax and code conversion
    __builtin_amdgcn_s_setprio(1);
    f32x4 sacc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      sacc[cb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(&S.t.kt[16 * cb + m][32 * ks + kq]);
        sacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qh[ks]),
                                                           __builtin_bit_cast(bf16x8_t, fb), sacc[cb], 0, 0, 0);
        sacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ql[ks]),
                                                           __builtin_bit_cast(bf16x8_t, fb), sacc[cb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // scores, mask, online softmax
    auto softmax_tile = [&](auto masked_c) {
      constexpr bool kMasked = decltype(masked_c)::value;
      float sc[4][4];
      float tmax[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax[i] = kNegInf;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int tk = 16 * cb + m, t = t0 + tk;
        const float sk = S.ks[tk], zk = S.kz[tk];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = __builtin_fmaf(sk, sacc[cb][i], zk * qs[i]);
          sc[cb][i] = (!kMasked || t <= prow[i]) ? v : kNegInf;
          tmax[i] = fmaxf(tmax[i], sc[cb][i]);
        }
      }
      float alpha[4], mnew[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = tmax[i];
        x = fmaxf(x, __shfl_xor(x, 1));
        x = fmaxf(x, __shfl_xor(x, 2));
        x = fmaxf(x, __shfl_xor(x, 4));
        x = fmaxf(x, __shfl_xor(x, 8));
        mnew[i] = fmaxf(mrun[i], x);
        // unmasked: mnew is finite, and exp2(-inf) = 0 covers a first tile
        alpha[i] = (kMasked && mnew[i] == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(mrun[i] - mnew[i]);
        mrun[i] = mnew[i];
        lrun[i] *= alpha[i];
        zrun[i] *= alpha[i];
      }
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[db][i] *= alpha[i];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int tk = 16 * cb + m;
        const float sv = S.vs[tk], zv = S.vz[tk];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * wave + 4 * (lane >> 4) + i;
          const float p = (kMasked && sc[cb][i] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sc[cb][i] - mnew[i]);
          lrun[i] += p;
          zrun[i] = __builtin_fmaf(p, zv, zrun[i]);
          S.t.pf[r][tk] = p * sv;
        }
      }
    };
    if (t0 + 63 <= p_min)
      softmax_tile(std::integral_constant<bool, false>{});
    else
      softmax_tile(std::integral_constant<bool, true>{});
    // each wave reads back only the rows of p s_V it wrote, so no block
    // barrier is needed: an LDS wait and a wave barrier order the lanes
    wave_lds_sync();
    __builtin_amdgcn_s_setprio(1);
    // O += (p s_V) V: A = rows of p s_V (tokens 32 ks + kq .. + 8), B = V^T
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(&S.t.pf[16 * wave + m][32 * ks + kq]);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(&S.t.pf[16 * wave + m][32 * ks + kq + 4]);
      u32x4_t ah, al;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t h0, l0, h1, l1;
        split_bf16(e < 2 ? p0[2 * e] : p1[2 * e - 4], h0, l0);
        split_bf16(e < 2 ? p0[2 * e + 1] : p1[2 * e - 3], h1, l1);
        ah[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        al[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(&S.t.vt[16 * db + m][32 * ks + kq]);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                           __builtin_bit_cast(bf16x8_t, fb), oacc[db], 0, 0, 0);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                           __builtin_bit_cast(bf16x8_t, fb), oacc[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- o' = (O + sum p z_V) / l, then o = o' R_V^T
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float l = lrun[i], z = zrun[i];
    l += __shfl_xor(l, 1); z += __shfl_xor(z, 1);
    l += __shfl_xor(l, 2); z += __shfl_xor(z, 2);
    l += __shfl_xor(l, 4); z += __shfl_xor(z, 4);
    l += __shfl_xor(l, 8); z += __shfl_xor(z, 8);
    lrun[i] = 1.0f / l;
    zrun[i] = z;
  }
  __syncthreads();                                // the tiles are consumed: rows[] is free
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S.rows[16 * wave + 4 * (lane >> 4) + i][16 * db + m] = (oacc[db][i] + zrun[i]) * lrun[i];
  __syncthreads();
  const int d = tid & 127, r0 = tid >> 7;
  if (a.absorb_v) {
    for (int k = 0; k < 32; ++k) {
      const int r = r0 + 2 * k, i = i0 + r / a.Gq;
      if (i < a.n && i < i0 + QB)
        store_prefill_out(a, (((size_t)b * a.n + i) * a.Hq + h * a.Gq + r % a.Gq) * D + d, S.rows[r][d]);
    }
    return;
  }
  float acc[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.0f;
  for (int e = 0; e < D; ++e) {
    const float re = a.rvT[e * D + d];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = __builtin_fmaf(S.rows[r0 + 2 * k][e], re, acc[k]);
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int r = r0 + 2 * k, i = i0 + r / a.Gq;
    if (i < a.n && i < i0 + QB)
      store_prefill_out(a, (((size_t)b * a.n + i) * a.Hq + h * a.Gq + r % a.Gq) * D + d, acc[k]);
  }
}

// head_dim 512.  Block = 4 waves, one (sequence, kv head) and 16 query rows
// (16 / Gq queries x the Gq heads of the kv head); wave w owns head-dim slice
// [128 w, 128 w + 128), which is quantization group w.  Per 32-token key tile:
//   - each wave stages its slice of the tile in its own part of shared memory
//     (K [token][dim], V transposed [dim][token], bf16 operands as at
//     head_dim 128, with its group's per-token scale and zero);
//   - each wave computes its slice's share of the scores, s_K,w (q_w . c_w) +
//     z_K,w (sum of q_w), on v_mfma_f32_16x16x32_bf16 with q in two bf16
//     pieces, and writes it to shared memory; after a block barrier every wave
//     adds the four shares in the same order, so the scores, the mask and the
//     online softmax are identical in the four waves;
//   - each wave accumulates its slice of O += (p s_V,w) V_w (p s_V,w in two
//     bf16 pieces) and its group's share of sum p z_V,w.
// Last, o' = O / l over the 512 dims, and o = o' R_V^T (or o' itself).
namespace {

struct alignas(16) PAWideSmem {
  union {
    float rows[16][516];           // q rows before the rotation; o' rows before the un-rotation
    struct {
      uint16_t kt[4][32][136];     // per wave: K slice tile [token][dim], bf16 bits
      uint16_t vt[4][128][40];     // per wave: V slice tile [dim][token], bf16 bits
      float sp[4][16][33];         // per wave: its slice's share of the scores [row][token]
      float pf[4][16][36];         // per wave: p s_V,w [row][token]
    } t;
  };
  float ks[4][32], kz[4][32], vs[4][32], vz[4][32];   // per group: scale and zero of the tile's tokens
  float qsum[4][16];                                   // per group and row: sum of q over the slice
};

// row r of a 16-row block -> query index (clamped to the last query)
__device__ inline int row_query16(const PrefillAttnArgs& a, int i0, int r) { return min(i0 + r / a.Gq, a.n - 1); }

}  // namespace

__global__ __launch_bounds__(256) void prefill_attn_wide_kernel(PrefillAttnArgs a) {
  constexpr int D = 512, TK = 32;
  __shared__ PAWideSmem S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's slice and group
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const int QB = 16 / a.Gq;                       // queries per block
  const int i0 = (int)blockIdx.y * QB;
  const int T = a.lens ? a.lens[b] : a.T;
  const int sink_end = min(a.N, T), rec_begin = max(a.N, T - a.M);

  // ---- q rows (bf16 -> fp32), rotation by R_K, scale x log2 e
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int r = idx >> 9, d = idx & 511;
    const int i = row_query16(a, i0, r), hq = h * a.Gq + r % a.Gq;
    S.rows[r][d] = bf16_to_f32(a.q[(((size_t)b * a.n + i) * a.Hq + hq) * D + d]);
  }
  __syncthreads();
  {
    // thread: dims tid and tid + 256 of every row; sums over e in order
    float acc[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int e = 0; e < D; ++e) {
      const float r0 = a.rk[(size_t)e * D + tid], r1 = a.rk[(size_t)e * D + tid + 256];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = S.rows[r][e];
        acc[0][r] = __builtin_fmaf(x, r0, acc[0][r]);
        acc[1][r] = __builtin_fmaf(x, r1, acc[1][r]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S.rows[r][tid] = acc[0][r] * a.scale_log2;
      S.rows[r][tid + 256] = acc[1][r] * a.scale_log2;
    }
  }
  __syncthreads();
  // A operands of the wave's slice: lane (m, kq) holds row m, dims
  // 128 w + 32 ks + kq .. + 8, as two bf16 pieces
  const int m = lane & 15, kq = 8 * (lane >> 4);
  u32x4_t qh[4], ql[4];
  float qpart = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t h0, l0, h1, l1;
      split_bf16(S.rows[m][128 * w + 32 * ks + kq + 2 * e], h0, l0);
      split_bf16(S.rows[m][128 * w + 32 * ks + kq + 2 * e + 1], h1, l1);
      qh[ks][e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      ql[ks][e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      qpart += (bf16_to_f32(h0) + bf16_to_f32(l0)) + (bf16_to_f32(h1) + bf16_to_f32(l1));
    }
  }
  qpart += __shfl_xor(qpart, 16);
  qpart += __shfl_xor(qpart, 32);
  if (lane < 16) S.qsum[w][m] = qpart;
  wave_lds_sync();
  // accumulator layout: register i of a 16 x 16 block is row 4 (lane >> 4) + i,
  // column 16 cb + (lane & 15)
  float qs[4];
  int prow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qs[i] = S.qsum[w][4 * (lane >> 4) + i];
    prow[i] = T - a.n + row_query16(a, i0, 4 * (lane >> 4) + i);
  }
  __syncthreads();                                // rows[] is reused by the tiles
  const int p_max = T - a.n + min(i0 + QB - 1, a.n - 1);
  const int p_min = T - a.n + i0;
  const int ntiles = p_max / TK + 1;
  float mrun[4], lrun[4], zrun[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrun[i] = kNegInf;
    lrun[i] = 0.0f;
    zrun[i] = 0.0f;
  }
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0, 0, 0, 0};

  const PlaneDev& K = a.k;
  const PlaneDev& V = a.v;
  auto half_f32 = [](uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); };
  auto window = [&](int t) { return t < sink_end || t >= rec_begin; };
  auto win_src = [&](const PlaneDev& P, int t) -> const uint16_t* {
    return P.is_bf16 ? P.full + row_offset(bh, a.cap, t, D)
           : t < sink_end ? P.sink + row_offset(bh, a.N, t, D)
                          : P.ring + row_offset(bh, a.M, t % a.M, D);
  };
  for (int tt = 0; tt < ntiles; ++tt) {
    const int t0 = tt * TK;
    // ---- stage the wave's slice (the wave's previous PV reads are done:
    // its own shared-memory reads complete before these writes are issued)
    wave_lds_sync();
    {
      // K: lane (token tk = lane / 2, half kh) writes dims [64 kh, 64 kh + 64)
      // of the slice for token t0 + tk
      const int tk = lane >> 1, kh = lane & 1, t = t0 + tk;
      uint16_t* dst = &S.t.kt[w][tk][64 * kh];
      float sk = 0.0f, zk = 0.0f;
      if (t >= T) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(dst + 8 * i) = u32x4_t{0, 0, 0, 0};
      } else if (K.is_bf16 || window(t)) {
        const uint16_t* src = win_src(K, t) + 128 * w + 64 * kh;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4_t*>(dst + 8 * i) = *reinterpret_cast<const u32x4_t*>(src + 8 * i);
        sk = 1.0f;
      } else {
        const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(K.codes + kcode_byte(bh, a.cap, t, 32 * w + 16 * kh, D));
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(dst + 8 * i) = codes8_bf16(cw[i >> 1] >> (16 * (i & 1)));
        const uint32_t mw = K.meta[meta_index(bh, a.cap, t, w, D)];
        sk = half_f32(mw & 0xFFFFu);
        zk = half_f32(mw >> 16);
      }
      if (kh == 0) {
        S.ks[w][tk] = sk;
        S.kz[w][tk] = zk;
      }
    }
    {
      // V codes: lane = record l of the slice's 64-token code tile; it writes
      // dims l and l + 64 of the tile's 32 tokens (the tile's first or second
      // half of tokens, bytes 0-15 or 16-31 of every record: groups of 8
      // tokens G, record bytes 2 k + dh carry tokens 8 (k / 2) + (k % 2) +
      // {0, 2, 4, 6} of dim l + 64 dh at bits {0, 2, 4, 6})
      const int l = lane, half = (t0 & 63) >> 5;
      if (!V.is_bf16) {
        const uint8_t* vtile = V.codes + vcode_tile_base(bh, a.cap, t0, w, D);
        const u32x4_t c = *reinterpret_cast<const u32x4_t*>(vtile + 1024 * half + 16 * l);
#pragma unroll
        for (int dh = 0; dh < 2; ++dh) {
#pragma unroll
          for (int G = 0; G < 4; ++G) {
            const int re = 4 * G + dh, ro = 4 * G + 2 + dh;
            const uint32_t be = (c[re >> 2] >> (8 * (re & 3))) & 0xFFu;
            const uint32_t bo = (c[ro >> 2] >> (8 * (ro & 3))) & 0xFFu;
            const uint32_t v = be | (bo << 16);
            u32x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = codes2_bf16((v >> (2 * e)) & 0x00030003u);
            *reinterpret_cast<u32x4_t*>(&S.t.vt[w][l + 64 * dh][8 * G]) = o;
          }
        }
      }
      if (lane < TK) {
        const int t = t0 + lane;
        float sv = 0.0f, zv = 0.0f;
        if (t < T) {
          if (V.is_bf16 || window(t)) {
            sv = 1.0f;
          } else {
            const uint32_t mw = V.meta[meta_index(bh, a.cap, t, w, D)];
            sv = half_f32(mw & 0xFFFFu);
            zv = half_f32(mw >> 16);
          }
        }
        S.vs[w][lane] = sv;
        S.vz[w][lane] = zv;
      }
    }
    const bool tile_has_window = V.is_bf16 || t0 < sink_end || t0 + TK > rec_begin || t0 + TK > T;   // uniform
    if (tile_has_window) {
      // V rows of window tokens (every token of a bf16 plane) overwrite their
      // columns; positions past T are zeroed.  Lane: token lane / 2, dims
      // [64 (lane % 2), + 64) of the slice.
      wave_lds_sync();                            // the code pass has written every column
      const int tk = lane >> 1, qd = lane & 1, t = t0 + tk;
      if (t >= T) {
#pragma unroll
        for (int e = 0; e < 64; ++e) S.t.vt[w][64 * qd + e][tk] = 0;
      } else if (V.is_bf16 || window(t)) {
        const uint16_t* src = win_src(V, t) + 128 * w + 64 * qd;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(src + 8 * i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S.t.vt[w][64 * qd + 8 * i + 2 * e][tk] = (uint16_t)(x[e] & 0xFFFFu);
            S.t.vt[w][64 * qd + 8 * i + 2 * e + 1][tk] = (uint16_t)(x[e] >> 16);
          }
        }
      }
    }
    wave_lds_sync();

    // ---- the slice's share of the scores
    f32x4 sacc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      sacc[cb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(&S.t.kt[w][16 * cb + m][32 * ks + kq]);
        sacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qh[ks]),
                                                           __builtin_bit_cast(bf16x8_t, fb), sacc[cb], 0, 0, 0);
        sacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ql[ks]),
                                                           __builtin_bit_cast(bf16x8_t, fb), sacc[cb], 0, 0, 0);
      }
    }
    __syncthreads();                              // every wave has read the previous tile's shares
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int tk = 16 * cb + m;
      const float sk = S.ks[w][tk], zk = S.kz[w][tk];
#pragma unroll
      for (int i = 0; i < 4; ++i) S.t.sp[w][4 * (lane >> 4) + i][tk] = __builtin_fmaf(sk, sacc[cb][i], zk * qs[i]);
    }
    __syncthreads();

    // ---- scores (the four shares in order), mask, online softmax
    auto softmax_tile = [&](auto masked_c) {
      constexpr bool kMasked = decltype(masked_c)::value;
      float sc[2][4], tmax[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax[i] = kNegInf;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int tk = 16 * cb + m, t = t0 + tk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * (lane >> 4) + i;
          const float v = ((S.t.sp[0][r][tk] + S.t.sp[1][r][tk]) + S.t.sp[2][r][tk]) + S.t.sp[3][r][tk];
          sc[cb][i] = (!kMasked || t <= prow[i]) ? v : kNegInf;
          tmax[i] = fmaxf(tmax[i], sc[cb][i]);
        }
      }
      float mnew[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = tmax[i];
        x = fmaxf(x, __shfl_xor(x, 1));
        x = fmaxf(x, __shfl_xor(x, 2));
        x = fmaxf(x, __shfl_xor(x, 4));
        x = fmaxf(x, __shfl_xor(x, 8));
        mnew[i] = fmaxf(mrun[i], x);
        const float alpha = (kMasked && mnew[i] == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(mrun[i] - mnew[i]);
        mrun[i] = mnew[i];
        lrun[i] *= alpha;
        zrun[i] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db][i] *= alpha;
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int tk = 16 * cb + m;
        const float sv = S.vs[w][tk], zv = S.vz[w][tk];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = (kMasked && sc[cb][i] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sc[cb][i] - mnew[i]);
          lrun[i] += p;
          zrun[i] = __builtin_fmaf(p, zv, zrun[i]);
          S.t.pf[w][4 * (lane >> 4) + i][tk] = p * sv;
        }
      }
    };
    if (t0 + TK - 1 <= p_min)
      softmax_tile(std::integral_constant<bool, false>{});
    else
      softmax_tile(std::integral_constant<bool, true>{});
    wave_lds_sync();

    // ---- O_w += (p s_V,w) V_w: A = rows of p s_V (tokens kq .. kq + 8), B = V_w^T
    {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(&S.t.pf[w][m][kq]);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(&S.t.pf[w][m][kq + 4]);
      u32x4_t ah, al;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t h0, l0, h1, l1;
        split_bf16(e < 2 ? p0[2 * e] : p1[2 * e - 4], h0, l0);
        split_bf16(e < 2 ? p0[2 * e + 1] : p1[2 * e - 3], h1, l1);
        ah[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        al[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(&S.t.vt[w][16 * db + m][kq]);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                           __builtin_bit_cast(bf16x8_t, fb), oacc[db], 0, 0, 0);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                           __builtin_bit_cast(bf16x8_t, fb), oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- o' = (O + sum p z_V) / l per slice, then o = o' R_V^T
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float l = lrun[i], z = zrun[i];
    l += __shfl_xor(l, 1); z += __shfl_xor(z, 1);
    l += __shfl_xor(l, 2); z += __shfl_xor(z, 2);
    l += __shfl_xor(l, 4); z += __shfl_xor(z, 4);
    l += __shfl_xor(l, 8); z += __shfl_xor(z, 8);
    lrun[i] = 1.0f / l;
    zrun[i] = z;
  }
  __syncthreads();                                // the tiles are consumed: rows[] is free
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) S.rows[4 * (lane >> 4) + i][128 * w + 16 * db + m] = (oacc[db][i] + zrun[i]) * lrun[i];
  __syncthreads();
  if (a.absorb_v) {
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int r = idx >> 9, d = idx & 511, i = i0 + r / a.Gq;
      if (i < a.n && i < i0 + QB)
        store_prefill_out(a, (((size_t)b * a.n + i) * a.Hq + h * a.Gq + r % a.Gq) * D + d, S.rows[r][d]);
    }
    return;
  }
  float acc[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int e = 0; e < D; ++e) {
    const float r0 = a.rvT[(size_t)e * D + tid], r1 = a.rvT[(size_t)e * D + tid + 256];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = S.rows[r][e];
      acc[0][r] = __builtin_fmaf(x, r0, acc[0][r]);
      acc[1][r] = __builtin_fmaf(x, r1, acc[1][r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + r / a.Gq;
    if (i < a.n && i < i0 + QB) {
      const size_t o = (((size_t)b * a.n + i) * a.Hq + h * a.Gq + r % a.Gq) * D;
      store_prefill_out(a, o + tid, acc[0][r]);
      store_prefill_out(a, o + tid + 256, acc[1][r]);
    }
  }
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.D == 512) {
    const int QB = 16 / a.Gq;
    dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)((a.n + QB - 1) / QB));
    hipLaunchKernelGGL(prefill_attn_wide_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int QB = 64 / a.Gq;
  dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)((a.n + QB - 1) / QB));
  hipLaunchKernelGGL(prefill_attn_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
