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
// Block = 4 waves, one (sequence, kv head), one 128-token chunk (two of the
// cache's 64-token tiles) and one 128-wide group: a 128 x 128 output tile with
// the operands of each reduction step staged in shared memory (details at the
// kernel).  The rotated tile goes through shared memory to the quantizer, one
// 64-token half at a time (one row per wave at a time, as in the one-token
// append), and the V code tile of each half's 64 tokens and 128 dims is
// assembled there and written whole (2 KiB), merging the bits of tokens
// stored before this chunk.
#include "append_impl.h"

namespace oscar {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Quantizer epilogue of one 64-token cache tile [t0, t0 + 64) of group g:
// rows in tile[64][132] (fp32, rotated), codes staged in codes[64][128].
// One row per wave at a time; lane owns dims lane and lane + 64 of the group
// (the one-token append's arithmetic).  Then the V code tile of those 64
// tokens and 128 dims (2 KiB) is assembled and written whole.  Returns the
// largest V scale stored (0 for K or bf16 planes).
__device__ float prefill_epilogue(const AppendArgs& a, const PlaneDev& P, float* dump, int bh, int b, int h, int g,
                                  int t0, float (*tile)[132], uint8_t (*codes)[128]) {
  const int D = a.D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float wsmax = 0.0f;
  for (int r = wave; r < 64; r += 4) {
    const int t = t0 + r;
    if (t < a.T_old || t >= a.T_new) continue;       // wave-uniform
    float x[2];
    x[0] = tile[r][lane] + 0.0f;
    x[1] = tile[r][lane + 64] + 0.0f;
    const int d0 = 128 * g + lane;
    if (dump) {
      const size_t base = (((size_t)b * a.n_new + (t - a.T_old)) * a.Hkv + h) * D;
      dump[base + d0] = x[0];
      dump[base + d0 + 64] = x[1];
    }
    if (P.is_bf16) {
      const size_t base = row_offset(bh, a.cap, t, D);
      P.full[base + d0] = f32_to_bf16(x[0]);
      P.full[base + d0 + 64] = f32_to_bf16(x[1]);
      continue;
    }
    if (t < a.N) {
      const size_t base = row_offset(bh, a.N, t, D);
      P.sink[base + d0] = f32_to_bf16(x[0]);
      P.sink[base + d0 + 64] = f32_to_bf16(x[1]);
    }
    if (a.M > 0 && t >= a.N && t >= a.T_new - a.M) {
      const size_t base = row_offset(bh, a.M, t % a.M, D);
      P.ring[base + d0] = f32_to_bf16(x[0]);
      P.ring[base + d0 + 64] = f32_to_bf16(x[1]);
    }
    const float mx = wave_max(fmaxf(x[0], x[1]));
    const float mn = wave_min(fminf(x[0], x[1]));
    const GroupQ q = group_params(mx, mn, P.clip);
    const uint32_t code[2] = {quant_code(x[0], q), quant_code(x[1], q)};
    if (lane == 0) P.meta[meta_index(bh, a.cap, t, g, D)] = q.packed;
    wsmax = fmaxf(wsmax, q.sf);
    if (!P.tiled) {
      store_canonical<2>(code, lane, [&](int w) {
        return reinterpret_cast<uint32_t*>(P.codes + kcode_byte(bh, a.cap, t, 32 * g + 4 * w, D));
      });
    } else {
      codes[r][lane] = (uint8_t)code[0];
      codes[r][lane + 64] = (uint8_t)code[1];
    }
  }
  if (P.is_bf16 || !P.tiled) return wsmax;
  __syncthreads();
  // V code tile of tokens [t0, t0 + 64), dims [128 g, 128 g + 128): 2 KiB, 8
  // bytes per thread.  Byte p: half p >> 10, lane record (p >> 4) & 63, record
  // byte rec = 16 half + (p & 15) holds dim 64 (rec & 1) + 4 (l >> 2) + (l & 3)
  // of the four tokens 8 (rec >> 2) + ((rec & 3) >> 1) + 2 (q & 1) + 4 (q >> 1)
  // (q = 0..3) at bits 2 q.  Tokens outside [T_old, T_new) keep their bits.
  uint8_t* vt = P.codes + vcode_tile_base(bh, a.cap, t0, g, D);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = 8 * tid + j;
    const int half = p >> 10, l = (p >> 4) & 63, rec = 16 * half + (p & 15);
    const int ds = 64 * (rec & 1) + 4 * (l >> 2) + (l & 3);
    const int tb0 = 8 * (rec >> 2) + ((rec & 3) >> 1);
    uint32_t byte = 0, keep = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tb = tb0 + 2 * (q & 1) + 4 * (q >> 1);
      const int t = t0 + tb;
      if (t >= a.T_old && t < a.T_new)
        byte |= (uint32_t)codes[tb][ds] << (2 * q);
      else
        keep |= 3u << (2 * q);
    }
    if (keep == 0xFFu) continue;          // no token of this chunk in the byte
    if (keep) byte |= vt[p] & keep;
    vt[p] = (uint8_t)byte;
  }
  return wsmax;
}

// Shared memory: the operand stage of one reduction step (A: 128 rows x 32
// k, B: 3 pieces x 128 columns x 32 k, bf16, rows padded to 40 elements so
// that 16 lanes reading 16 rows at one k offset hit distinct banks), reused
// after the product for one 64-row half of the rotated tile and its codes.
struct PrefillSmem {
  union {
    struct {
      uint16_t A[128][40];
      uint16_t B[3][128][40];
    } st;
    struct {
      float tile[64][132];
      uint8_t codes[64][128];
    } ep;
  };
  float smax[4];
};

// Block = 4 waves, one (sequence, kv head), one 128-token chunk (two of the
// cache's 64-token tiles) and one 128-wide group of K or V: a 128 x 128 output
// tile, the reduction over head_dim in steps of 32.  Each step's operands are
// loaded from memory by all 256 threads into registers (8 x 16 bytes each),
// written to shared memory, and read back by the waves: wave (wr, wc) owns rows
// [64 wr, 64 wr + 64) and columns [64 wc, 64 wc + 64), 4 x 4 accumulators of
// 16 x 16; 48 products per wave per step.  The next step's loads are in
// flight during this step's products.
// 3 waves per SIMD (160 registers): measured 8-15% faster than the
// unconstrained 2 waves (245 registers) at both head dims.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void append_prefill_kernel(AppendArgs a) {
  constexpr int KS = D / 32;           // reduction steps
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const int g = blockIdx.z >> 1;       // 128-wide group
  const bool isv = (blockIdx.z & 1) != 0;
  const int t0 = ((a.T_old >> 7) + (int)blockIdx.y) << 7;   // first position of the 128-token chunk
  const PlaneDev P = isv ? a.v : a.k;
  const uint16_t* in = isv ? a.vin : a.kin;
  const uint16_t* RT = isv ? a.rv3 : a.rk3;   // [3][D (column n)][D (row k)] bf16
  float* dump = isv ? a.vdump : a.kdump;
  __shared__ PrefillSmem S;

  // global -> register staging: A chunks j = tid, tid + 256 (row j >> 2, 16-byte
  // piece j & 3 of its 32 k); B chunks j = tid + 256 i, i < 6 (piece j / 512,
  // column (j >> 2) & 127, 16-byte piece j & 3)
  const uint16_t* asrc[2];
  bool aval[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = tid + 256 * i, row = j >> 2, t = t0 + row;
    aval[i] = t >= a.T_old && t < a.T_new;
    asrc[i] = in + ((((size_t)b * a.n_new + (aval[i] ? t - a.T_old : 0)) * a.Hkv + h) * D) + 8 * (j & 3);
  }
  const uint16_t* bsrc[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int j = tid + 256 * i, s = j >> 9, col = (j >> 2) & 127;
    bsrc[i] = RT + ((size_t)s * D + 128 * g + col) * D + 8 * (j & 3);
  }
  u32x4_t ra[2], rb_[6];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = aval[i] ? *reinterpret_cast<const u32x4_t*>(asrc[i] + k0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 6; ++i) rb_[i] = *reinterpret_cast<const u32x4_t*>(bsrc[i] + k0);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = tid + 256 * i;
      *reinterpret_cast<u32x4_t*>(&S.st.A[j >> 2][8 * (j & 3)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int j = tid + 256 * i;
      *reinterpret_cast<u32x4_t*>(&S.st.B[j >> 9][(j >> 2) & 127][8 * (j & 3)]) = rb_[i];
    }
  };

  const int wr = wave >> 1, wc = wave & 1;
  const int m = lane & 15, kq = 8 * (lane >> 4);
  f32x4 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0, 0, 0, 0};

  gload(0);
  sstore();
  __syncthreads();
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) gload(32 * (ks + 1));
    u32x4_t fa[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) fa[rb] = *reinterpret_cast<const u32x4_t*>(&S.st.A[64 * wr + 16 * rb + m][kq]);
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(&S.st.B[s][64 * wc + 16 * cb + m][kq]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[rb]),
                                                                __builtin_bit_cast(bf16x8_t, fb), acc[rb][cb], 0, 0, 0);
      }
    __syncthreads();                     // every wave has read this step's operands
    if (ks + 1 < KS) {
      sstore();
      __syncthreads();
    }
  }

  // two halves of 64 rows (one cache tile each): accumulator (rb, cb)
  // register i is row 64 wr + 16 rb + 4 (lane >> 4) + i, column 64 wc + 16 cb + m
  if (tid < 4) S.smax[tid] = 0.0f;
  float wsmax = 0.0f;
  for (int half = 0; half < 2; ++half) {
    if (wr == half) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) S.ep.tile[16 * rb + 4 * (lane >> 4) + i][64 * wc + 16 * cb + m] = acc[rb][cb][i];
    }
    __syncthreads();
    const int th = t0 + 64 * half;
    if (th < a.T_new && th + 64 > a.T_old)
      wsmax = fmaxf(wsmax, prefill_epilogue(a, P, dump, bh, b, h, g, th, S.ep.tile, S.ep.codes));
    __syncthreads();                     // the tile and codes are rewritten by the next half
  }
  if (P.smax && lane == 0 && wsmax > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(&S.smax[0]), __float_as_uint(wsmax));
  __syncthreads();
  if (P.smax && tid == 0 && S.smax[0] > 0.0f)
    atomicMax(reinterpret_cast<unsigned int*>(P.smax + bh), __float_as_uint(S.smax[0]));
}

hipError_t launch_append_prefill(const AppendArgs& a, hipStream_t s) {
  const int tiles = ((a.T_new - 1) >> 7) - (a.T_old >> 7) + 1;   // 128-token chunks
  dim3 grid((unsigned)(a.batch * a.Hkv), (unsigned)tiles, (unsigned)(2 * (a.D / 128)));
  if (a.D == 128)
    hipLaunchKernelGGL(append_prefill_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_prefill_kernel<512>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
