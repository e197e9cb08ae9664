// Multi-token append (chunked prefill) with the rotation on matrix cores.
//
// The append path rotates every new K and V row by the layer's R_K / R_V,
// then clips, quantizes to 2 bits and packs each 128-wide group ("OSCAR: 2-bit
// KV Cache Quantization for SGLang and llama.cpp", "How the offline rotation
// is fit"; the clip ratios and group size in the Qwen3-4B card's "Run" table).
// For a prefill chunk the rotation is a dense product X (rows = tokens) times
// R (head_dim x head_dim), done here with v_mfma_f32_16x16x32_bf16:
//
//   X is bf16 already, so it enters the matrix cores unchanged.  R is fp32;
//   it is held as three bf16 matrices R = R1 + R2 + R3 (R1 = bf16(R), R2 =
//   bf16(R - R1), R3 = R - R1 - R2, which is exact for every finite fp32 R
//   outside the subnormal range).  Each product of a bf16 x and a bf16 piece
//   is exact in fp32, so X R is computed in fp32 with only the accumulation
//   order differing from a plain fp32 loop.
//
// Block = 4 waves, one (sequence, kv head), 256 tokens (four of the cache's
// 64-token tiles) and one 128-wide group: a 256 x 128 output tile (details at
// the kernel).  The rotated tile goes through shared memory to the quantizer,
// one 64-token quarter at a time, four lanes per token row, and the V code
// tile of each quarter's 64 tokens and 128 dims is assembled there and written
// whole (2 KiB), merging the bits of tokens stored before this chunk.
#include "append_impl.h"

namespace oscar {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRawBuffer = 0x00020000;   // buffer resource config: raw 32-bit data, no swizzle

// max / min of a value over the 4 lanes of a quad (lanes 4i .. 4i + 3), through
// DPP quad permutations (xor 1, then xor 2).
__device__ inline float quad_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  return v;
}
__device__ inline float quad_min(float v) {
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  return v;
}

__device__ inline float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}

// Sum of a 128-value group held by a quad (lane p: values [32 p, 32 p + 32))
// in the pairwise order of group_sum128: value i with i + 64 (lanes p and
// p ^ 2), then with i + 32 (lanes p and p ^ 1), then the in-lane halves.
__device__ inline float quad_sum128(const float (&x)[32]) {
  float y[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = as_f32(x[j] + quad_xor2(x[j]));
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = as_f32(y[j] + quad_xor1(y[j]));
#pragma unroll
  for (int h = 16; h >= 1; h >>= 1)
#pragma unroll
    for (int j = 0; j < h; ++j) y[j] = as_f32(y[j] + y[j + h]);
  return y[0];
}

// Quantizer epilogue of one 64-token cache tile [t0, t0 + 64) of group g: the
// rotated rows are in tile[64][132] (fp32).  Four lanes per row (thread tid:
// row tid / 4, quad lane p = tid % 4); lane p takes the row's values [32 p,
// 32 p + 32) for everything:
//   - the fp32 dump, the bf16 windows and the bf16 plane;
//   - the group's max and min (in-lane, then two DPP steps over the quad), the
//     one-token append's arithmetic for scale and zero, and the codes of its
//     32 values, which are canonical words 2 p and 2 p + 1 of the row (code of
//     value e at bit 2 (e % 16) of word e / 16), so no lane exchange is needed.
// For V the packed rows go to crow[64][8] in shared memory, and the V code
// tile of those 64 tokens and 128 dims (2 KiB) is assembled from them and
// written whole.  Rows outside [T_old, T_new) are computed (their tile rows are
// finite) but nothing of them is stored.  Returns this lane's largest stored V
// scale (0 for K or bf16 planes).
template <bool LM>
__device__ float prefill_epilogue(const AppendArgs& a, const PlaneDev& P, float* dump, int bh, int b, int h, int g,
                                  int t0, int T_old, int T_new, float (*tile)[132], uint32_t (*crow)[8]) {
  const int D = a.D;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const int t = t0 + r;
  const bool live = t >= T_old && t < T_new;
  const int d0 = 128 * g;
  float x[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&tile[r][32 * p + 4 * i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = v[e] + 0.0f;   // -0 -> +0
  }
  const bool to_full = P.is_bf16;
  const bool to_sink = !P.is_bf16 && t < a.N;
  const bool to_ring = !P.is_bf16 && a.M > 0 && t >= a.N && t >= T_new - a.M;
  if (live && dump) {
    float* drow = dump + (((size_t)b * a.n_new + (t - T_old)) * a.Hkv + h) * D + d0 + 32 * p;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<f32x4*>(drow + 4 * i) = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
  }
  if (live && (to_full || to_sink || to_ring)) {
    // a position in the sink is never in the ring (t >= N there); a bf16 plane
    // has no windows
    uint16_t* wrow = to_full ? P.full + row_offset(bh, a.cap, t, D)
                   : to_sink ? P.sink + row_offset(bh, a.N, t, D)
                             : P.ring + row_offset(bh, a.M, t % a.M, D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)f32_to_bf16(x[8 * i + 2 * e]) | ((uint32_t)f32_to_bf16(x[8 * i + 2 * e + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(wrow + d0 + 32 * p + 8 * i) = w;
    }
  }
  if (P.is_bf16) return 0.0f;

  GroupQ q;
  uint32_t w0 = 0, w1 = 0;
  if constexpr (LM) {
    const float mean = as_f32(quad_sum128(x) * 0.0078125f);
    float dd[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float d = as_f32(x[j] - mean);
      dd[j] = as_f32(d * d);
    }
    q = lm_group_params(mean, quad_sum128(dd), P.clip);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      w0 |= lm_code(x[j], q) << (2 * j);
      w1 |= lm_code(x[16 + j], q) << (2 * j);
    }
  } else {
    float mx = x[0], mn = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
      mx = fmaxf(mx, x[j]);
      mn = fminf(mn, x[j]);
    }
    mx = quad_max(mx);
    mn = quad_min(mn);
    q = group_params(mx, mn, P.clip);
    const float inv = __builtin_amdgcn_rcpf(q.sf);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      w0 |= quant_code_fast(x[j], q, inv) << (2 * j);
      w1 |= quant_code_fast(x[16 + j], q, inv) << (2 * j);
    }
  }
  float smax = 0.0f;
  if (live) {
    if (p == 0) P.meta[meta_index(bh, a.cap, t, g, D)] = q.packed;
    smax = q.sf;
    if (!P.tiled) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2_t*>(P.codes + kcode_byte(bh, a.cap, t, 32 * g + 8 * p, D)) = u32x2_t{w0, w1};
    }
  }
  if (!P.tiled) return 0.0f;
  crow[r][2 * p] = w0;
  crow[r][2 * p + 1] = w1;
  __syncthreads();
  // V code tile of tokens [t0, t0 + 64), dims [128 g, 128 g + 128): 2 KiB, 8
  // bytes per thread.  Byte p8: half p8 >> 10, lane record (p8 >> 4) & 63, record
  // byte rec = 16 half + (p8 & 15) holds dim 64 (rec & 1) + 4 (l >> 2) + (l & 3)
  // of the four tokens 8 (rec >> 2) + ((rec & 3) >> 1) + 2 (qq & 1) + 4 (qq >> 1)
  // (qq = 0..3) at bits 2 qq.  Tokens outside [T_old, T_new) keep their bits.
  uint8_t* vt = P.codes + vcode_tile_base(bh, a.cap, t0, g, D);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p8 = 8 * tid + j;
    const int half = p8 >> 10, l = (p8 >> 4) & 63, rec = 16 * half + (p8 & 15);
    const int ds = 64 * (rec & 1) + 4 * (l >> 2) + (l & 3);
    const int tb0 = 8 * (rec >> 2) + ((rec & 3) >> 1);
    uint32_t byte = 0, keep = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int tb = tb0 + 2 * (qq & 1) + 4 * (qq >> 1);
      const int tt = t0 + tb;
      if (tt >= T_old && tt < T_new)
        byte |= ((crow[tb][ds >> 4] >> (2 * (ds & 15))) & 3u) << (2 * qq);
      else
        keep |= 3u << (2 * qq);
    }
    if (keep == 0xFFu) continue;          // no token of this chunk in the byte
    if (keep) byte |= vt[p8] & keep;
    vt[p8] = (uint8_t)byte;
  }
  return smax;
}

// Shared memory: two stages of the B operand (3 pieces x 128 columns x 32 k of
// R^T, bf16, rows padded to 40 elements so that 16 lanes reading 16 columns at
// one k offset hit distinct banks), reused after the product for one 64-row
// quarter of the rotated tile and its packed code rows.
struct PrefillSmem {
  union {
    uint16_t B[2][3][128][40];
    struct {
      float tile[64][132];
      uint32_t crow[64][8];
    } ep;
  };
  float smax[4];
};

// Block = 4 waves, one (sequence, kv head), 256 tokens (four of the cache's
// 64-token tiles) and one 128-wide group of K or V: a 256 x 128 output tile,
// the reduction over head_dim in steps of 32.  Wave w owns rows [64 w, 64 w +
// 64) and all 128 columns: 4 x 8 accumulators of 16 x 16, 96 products per
// step.  A (the bf16 input rows) goes straight from memory into the lanes'
// operand registers; B (the three pieces of R) is staged through shared memory
// in two alternating buffers, so each step has one barrier.  Both operands of
// step ks + 1 are in flight during step ks.
//
// Placement: the dispatcher deals blocks to the 8 XCDs in turn (block i to XCD
// i mod 8), each with its own L2.  At head_dim 512 the four groups of a row
// tile read the same input rows, so the block index is remapped to give the
// four groups of one row tile consecutive slots on the same XCD: the rows come
// from HBM once and from that L2 three times.
template <int D, bool LM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void append_prefill_kernel(
    AppendArgs a, int row_tiles, int tiles_per_bh) {
  constexpr int KS = D / 32;           // reduction steps
  constexpr int NG = D / 128;          // groups
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = blockIdx.x, xcd = L & 7, r = L >> 3;
  const int rt = (r / NG) * 8 + xcd;   // row tile: (K or V, sequence, kv head, 256-token tile)
  const int g = r - (r / NG) * NG;
  if (rt >= row_tiles) return;         // padding of the last round of 8
  const int isv_i = rt / (a.batch * a.Hkv * tiles_per_bh);
  const int rem = rt - isv_i * (a.batch * a.Hkv * tiles_per_bh);
  const int bh = rem / tiles_per_bh, y = rem - (rem / tiles_per_bh) * tiles_per_bh;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const bool isv = isv_i != 0;
  const int2 tr = append_range(a, b);         // this sequence's new positions [tr.x, tr.y)
  const int t0 = ((tr.x >> 8) + y) << 8;      // first position of the 256-token tile
  if (t0 >= tr.y) return;                     // ragged batch: this sequence has fewer tiles
  const PlaneDev P = isv ? a.v : a.k;
  const uint16_t* in = isv ? a.vin : a.kin;
  const uint16_t* RT = isv ? a.rv3 : a.rk3;   // [3][D (column n)][D (row k)] bf16
  float* dump = isv ? a.vdump : a.kdump;
  __shared__ PrefillSmem S;

  // Operands are read through buffer resources: one uniform base, a 32-bit
  // lane offset and a uniform step offset, so the loads hold few registers.
  // A: the lane's rows 64 wave + 16 rb + m, k offset kq within each step.
  // Rows outside [tr.x, tr.y) read the first new row instead (always present): their
  // products are never stored (each output row depends on its own A row
  // only), and unconditional loads keep the wait counts static.
  const int m = lane & 15, kq = 8 * (lane >> 4);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(in + (size_t)b * a.n_new * a.Hkv * D), (short)0, a.n_new * a.Hkv * D * 2, kRawBuffer);
  int aoff[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int t = t0 + 64 * wave + 16 * rb + m;
    const int row = (t >= tr.x && t < tr.y) ? t - tr.x : 0;
    aoff[rb] = ((row * a.Hkv + h) * D + kq) * 2;
  }
  // B staging: chunks i < 6 of 16 bytes per thread: piece i >> 1, column
  // (tid >> 2) + 64 (i & 1) of group g, 16-byte piece tid & 3 of the step's 32 k
  const __amdgpu_buffer_rsrc_t brsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(RT), (short)0, 3 * D * D * 2, kRawBuffer);
  const int boff = ((128 * g + (tid >> 2)) * D + 8 * (tid & 3)) * 2;
  u32x4_t rbs[6];
  auto bload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 6; ++i)
      rbs[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               brsrc, boff, ((i >> 1) * D * D + 64 * (i & 1) * D + k0) * 2, 0));
  };
  auto bstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 6; ++i)
      *reinterpret_cast<u32x4_t*>(&S.B[buf][i >> 1][(tid >> 2) + 64 * (i & 1)][8 * (tid & 3)]) = rbs[i];
  };
  auto aload = [&](u32x4_t (&dst)[4], int k0) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      dst[rb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[rb], k0 * 2, 0));
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[rb][cb] = f32x4{0, 0, 0, 0};

  // step ks: products from buffer ks & 1 and the A registers ra; stores B of
  // step ks + 1 (loaded during step ks - 1) into the other buffer, then issues
  // the loads of step ks + 2, A into the registers this step has consumed.
  // The loads are unconditional (the last two steps reload the last step's
  // operands, unused) and scheduling barriers keep each phase in place, so the
  // wait counts stay static: the B store waits for B only, the products for
  // their own A only.
  auto step = [&](int ks, u32x4_t (&ra)[4]) {
    const int buf = ks & 1;
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(&S.B[buf][s][16 * cb + m][kq]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ra[rb]),
                                                                __builtin_bit_cast(bf16x8_t, fb), acc[rb][cb], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    bstore(buf ^ 1);
    __syncthreads();                     // buffer buf ^ 1 is complete; buffer buf is free
    __builtin_amdgcn_sched_barrier(0);
    const int k2 = 32 * min(ks + 2, KS - 1);
    bload(k2);
    aload(ra, k2);
    __builtin_amdgcn_sched_barrier(0);
  };

  u32x4_t ra0[4], ra1[4];
  bload(0);
  aload(ra0, 0);
  bstore(0);
  __syncthreads();
  bload(32);
  aload(ra1, 32);
  // KS is even (4 or 16): steps alternate between the two A register sets
#pragma unroll 1
  for (int ks = 0; ks < KS; ks += 2) {
    step(ks, ra0);
    step(ks + 1, ra1);
  }

  // four quarters of 64 rows (one cache tile each): accumulator (rb, cb)
  // register i of wave w is row 64 w + 16 rb + 4 (lane >> 4) + i, column 16 cb + m
  if (tid < 4) S.smax[tid] = 0.0f;
  float wsmax = 0.0f;
  for (int qt = 0; qt < 4; ++qt) {
    const int th = t0 + 64 * qt;
    const bool live = th < tr.y && th + 64 > tr.x;          // block-uniform
    if (!live) continue;
    if (wave == qt) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) S.ep.tile[16 * rb + 4 * (lane >> 4) + i][16 * cb + m] = acc[rb][cb][i];
    }
    __syncthreads();
    wsmax = fmaxf(wsmax, prefill_epilogue<LM>(a, P, dump, bh, b, h, g, th, tr.x, tr.y, S.ep.tile, S.ep.crow));
    __syncthreads();                     // the tile and codes are rewritten by the next quarter
  }
  wsmax = wave_max(wsmax);
  if (P.smax && lane == 0 && wsmax > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(&S.smax[0]), __float_as_uint(wsmax));
  __syncthreads();
  if (P.smax && tid == 0 && S.smax[0] > 0.0f)
    atomicMax(reinterpret_cast<unsigned int*>(P.smax + bh), __float_as_uint(S.smax[0]));
}

hipError_t launch_append_prefill(const AppendArgs& a, hipStream_t s) {
  // the input of one sequence is addressed with 32-bit byte offsets
  if ((long long)a.n_new * a.Hkv * a.D * 2 > INT32_MAX) return hipErrorInvalidValue;
  const int tiles = ((a.T_new - 1) >> 8) - (a.T_old >> 8) + 1;   // 256-token tiles per (sequence, kv head)
  const int row_tiles = 2 * a.batch * a.Hkv * tiles;
  const int ng = a.D / 128;
  const unsigned blocks = (unsigned)((row_tiles + 7) / 8) * 8u * (unsigned)ng;
  const bool lm = a.k.lm != 0;
  if (a.D == 128) {
    if (lm)
      hipLaunchKernelGGL((append_prefill_kernel<128, true>), dim3(blocks), dim3(256), 0, s, a, row_tiles, tiles);
    else
      hipLaunchKernelGGL((append_prefill_kernel<128, false>), dim3(blocks), dim3(256), 0, s, a, row_tiles, tiles);
  } else {
    if (lm)
      hipLaunchKernelGGL((append_prefill_kernel<512, true>), dim3(blocks), dim3(256), 0, s, a, row_tiles, tiles);
    else
      hipLaunchKernelGGL((append_prefill_kernel<512, false>), dim3(blocks), dim3(256), 0, s, a, row_tiles, tiles);
  }
  return hipGetLastError();
}

}  // namespace oscar
