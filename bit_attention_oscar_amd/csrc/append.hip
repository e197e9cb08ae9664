// Append path: rotate, write the bf16 window copy, clip + INT2-quantize + pack.
// Built with -ffp-contract=off and correctly rounded fp32 division so the
// quantizer performs exactly one IEEE rounding per operation.
//
// Method (web pages on OSCAR): rotation of post-RoPE K and V by one orthogonal
// head_dim x head_dim matrix per layer ("OSCAR-LLAMACPP-Qwen3-4B-Thinking-2507-
// INT2-KV", "Files" note; "OSCAR-RotationZoo", "File format"); clip before
// quantization (Qwen3-4B card, "Run" env-var table; K 0.96 / V 0.92 in the
// RotationZoo card, "How to use" step 2); INT2 with group 128 along head_dim
// (RotationZoo card, same flags); bf16 sink and recent window (Qwen3-4B card,
// "Run" table; "OSCAR: 2-bit KV Cache Quantization for SGLang and llama.cpp",
// "What OSCAR compresses").
#include <algorithm>
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

// Canonical packing through lane shuffles: lane l holds the code of dim
// l + 64 i; word w (dims 16w..16w+15) is OR-reduced over the 16 lanes
// 16 (w % 4) .. + 15 of element i = w / 4 and stored by its first lane.
template <int PER>
__device__ inline void store_canonical(const uint32_t* code, int lane, uint8_t* row) {
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    uint32_t v = code[i] << (2 * (lane & 15));
    v |= __shfl_xor(v, 1);
    v |= __shfl_xor(v, 2);
    v |= __shfl_xor(v, 4);
    v |= __shfl_xor(v, 8);
    if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(row + 4 * (4 * i + (lane >> 4))) = v;
  }
}

// Block per (sequence, kv head, 8-token group); blockIdx.z: 0 = K, 1 = V.
// NT token slots (1 for a one-token append, 8 otherwise).  The reduction over
// e of the rotation is split across WAVES waves (partial sums added in a fixed
// order); wave 0 then quantizes and stores.  Wave 0's lane l owns dims
// l + 64 i, so it also owns the V tile bytes of those dims for every token of
// the group (tiled-layout bytes are shared only among tokens of one group of
// 8 at one dim, and one block handles the whole group).
template <int D, int WAVES, int NT>
__global__ __launch_bounds__(64 * WAVES) void append_kernel(AppendArgs a) {
  constexpr int PER = D / 64;
  constexpr int EW = D / WAVES;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh - (bh / a.Hkv) * a.Hkv;
  const bool isv = blockIdx.z != 0;
  const PlaneDev P = isv ? a.v : a.k;
  const uint16_t* in = isv ? a.vin : a.kin;
  const float* R = isv ? a.rv : a.rk;
  float* dump = isv ? a.vdump : a.kdump;
  const int g8 = (a.T_old >> 3) + (int)blockIdx.y;
  const int t_lo = NT == 1 ? a.T_old : max(a.T_old, g8 * 8);
  const int t_hi = NT == 1 ? a.T_old + 1 : min(a.T_new, g8 * 8 + 8);
  const int ntok = t_hi - t_lo;

  __shared__ float xs[NT][D];
  __shared__ float part[WAVES][NT][D];
  for (int i = tid; i < NT * D; i += 64 * WAVES) {
    const int tk = i / D, d = i - (i / D) * D;
    float v = 0.0f;
    if (tk < ntok) {
      const int t = t_lo + tk;
      const size_t idx = (((size_t)b * a.n_new + (t - a.T_old)) * a.Hkv + h) * D + d;
      v = bf16_to_f32(in[idx]);
    }
    xs[tk][d] = v;
  }
  __syncthreads();

  // partial x_rot[d] = sum over this wave's e of x[e] * R[e][d], e ascending
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
      const float x = xs[tk][wave * EW + e];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[tk][i] = __builtin_fmaf(x, r[i], acc[tk][i]);
    }
  }
  if (WAVES > 1) {
#pragma unroll
    for (int tk = 0; tk < NT; ++tk)
#pragma unroll
      for (int i = 0; i < PER; ++i) part[wave][tk][lane + 64 * i] = acc[tk][i];
    __syncthreads();
    if (wave != 0) return;
  }

#pragma unroll
  for (int tk = 0; tk < NT; ++tk) {
    if (tk >= ntok) break;
    const int t = t_lo + tk;
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float v = acc[tk][i];
      if (WAVES > 1) {
        const int d = lane + 64 * i;
        v = part[0][tk][d];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v = v + part[w][tk][d];
      }
      x[i] = v + 0.0f;   // -0 -> +0
    }
    if (dump) {
      const size_t base = (((size_t)b * a.n_new + (t - a.T_old)) * a.Hkv + h) * D;
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
      for (int i = 0; i < PER; ++i) P.sink[base + lane + 64 * i] = f32_to_bf16(x[i]);
    }
    if (a.M > 0 && t >= a.N && t >= a.T_new - a.M) {
      const size_t base = row_offset(bh, a.M, t % a.M, D);
#pragma unroll
      for (int i = 0; i < PER; ++i) P.ring[base + lane + 64 * i] = f32_to_bf16(x[i]);
    }
    uint32_t code[PER];
#pragma unroll
    for (int g = 0; g < D / kGroup; ++g) {
      // group g = dims [128 g, 128 g + 128) = elements 2g, 2g+1 of every lane
      const float mx = wave_max(fmaxf(x[2 * g], x[2 * g + 1]));
      const float mn = wave_min(fminf(x[2 * g], x[2 * g + 1]));
      const GroupQ q = group_params(mx, mn, P.clip);
      code[2 * g] = quant_code(x[2 * g], q);
      code[2 * g + 1] = quant_code(x[2 * g + 1], q);
      if (lane == 0) {
        P.meta[meta_offset(bh, a.cap, t, D) + g] = q.packed;
        if (P.smax) atomicMax(reinterpret_cast<unsigned int*>(P.smax + bh), __float_as_uint(q.sf));
      }
    }
    if (!P.tiled) {
      store_canonical<PER>(code, lane, P.codes + kcode_offset(bh, a.cap, t, D));
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int bit;
        const size_t off = vcode_byte(bh, a.cap, t, lane + 64 * i, D, &bit);
        const uint8_t old = P.codes[off];
        P.codes[off] = (uint8_t)((old & ~(3u << bit)) | (code[i] << bit));
      }
    }
  }
}

// Test hook: the same quantizer on fp32 rows, canonical packing.
template <int D>
__global__ __launch_bounds__(64) void quantize_rows_kernel(const float* x, float clip, uint8_t* codes,
                                                           uint32_t* meta) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = x[row * D + lane + 64 * i] + 0.0f;
  uint32_t code[PER];
#pragma unroll
  for (int g = 0; g < D / kGroup; ++g) {
    const float mx = wave_max(fmaxf(v[2 * g], v[2 * g + 1]));
    const float mn = wave_min(fminf(v[2 * g], v[2 * g + 1]));
    const GroupQ q = group_params(mx, mn, clip);
    code[2 * g] = quant_code(v[2 * g], q);
    code[2 * g + 1] = quant_code(v[2 * g + 1], q);
    if (lane == 0) meta[row * (D / kGroup) + g] = q.packed;
  }
  store_canonical<PER>(code, lane, codes + row * (D / 4));
}

// Canonical export of the tiled V codes: one thread per output byte.
__global__ __launch_bounds__(256) void export_vcodes_kernel(const uint8_t* tiled, uint8_t* canon, int BH,
                                                            int cap, int T, int D) {
  const size_t nbytes = (size_t)BH * T * (D / 4);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nbytes;
       i += (size_t)gridDim.x * blockDim.x) {
    const int byte = (int)(i % (D / 4));
    const size_t rowi = i / (D / 4);
    const int t = (int)(rowi % T);
    const int bh = (int)(rowi / T);
    uint32_t out = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int bit;
      const size_t off = vcode_byte(bh, cap, t, 4 * byte + k, D, &bit);
      out |= (uint32_t)((tiled[off] >> bit) & 3u) << (2 * k);
    }
    canon[i] = (uint8_t)out;
  }
}

// Plain 16-byte copy used to calibrate bandwidth and traffic counters.
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4* src, uint4* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int groups = ((a.T_new - 1) >> 3) - (a.T_old >> 3) + 1;
  dim3 grid((unsigned)(a.batch * a.Hkv), (unsigned)groups, 2);
  const bool one = a.n_new == 1;
  if (a.D == 128) {
    if (one)
      hipLaunchKernelGGL((append_kernel<128, 4, 1>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<128, 4, 8>), grid, dim3(256), 0, s, a);
  } else {
    if (one)
      hipLaunchKernelGGL((append_kernel<512, 4, 1>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<512, 1, 8>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* x, int rows, int D, float clip, uint8_t* codes,
                                uint32_t* meta, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(quantize_rows_kernel<128>, dim3(rows), dim3(64), 0, s, x, clip, codes, meta);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<512>, dim3(rows), dim3(64), 0, s, x, clip, codes, meta);
  return hipGetLastError();
}

hipError_t launch_export_vcodes(const uint8_t* tiled, uint8_t* canon, int BH, int cap, int T, int D,
                                hipStream_t s) {
  const size_t n = (size_t)BH * T * (D / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(export_vcodes_kernel, dim3(blocks), dim3(256), 0, s, tiled, canon, BH, cap, T, D);
  return hipGetLastError();
}

}  // namespace oscar
