// Append kernels (rotate, bf16 window copy, clip + INT2-quantize + pack; the
// device code is in append_impl.h), the quantizer test hook, the canonical
// export of the tiled V codes and the copy calibration kernel.
#include <algorithm>
#include "append_impl.h"

namespace oscar {

// Block per (sequence, kv head, 8-token group); blockIdx.z: 0 = K, 1 = V.
// NT token slots (1 for a one-token append, 8 otherwise); the rotation's
// reduction over e is split across WAVES waves.
template <int D, int WAVES, int NT>
__global__ __launch_bounds__(64 * WAVES) void append_kernel(AppendArgs a) {
  __shared__ float xs[NT * D];
  __shared__ float part[WAVES * NT * D];
  const int2 tr = append_range(a, (int)blockIdx.x / a.Hkv);
  const int g8 = (tr.x >> 3) + (int)blockIdx.y;
  const int t_lo = NT == 1 ? tr.x : max(tr.x, g8 * 8);
  const int t_hi = NT == 1 ? tr.x + 1 : min(tr.y, g8 * 8 + 8);
  if (t_lo >= t_hi) return;            // ragged batch: this sequence has fewer 8-token groups
  if (a.k.lm)
    append_block<D, WAVES, NT, true>(a, (int)blockIdx.x, blockIdx.z != 0, t_lo, t_hi, tr.x, tr.y, xs, part);
  else
    append_block<D, WAVES, NT, false>(a, (int)blockIdx.x, blockIdx.z != 0, t_lo, t_hi, tr.x, tr.y, xs, part);
}

// One-token append at head_dim 512: grid (sequence x kv head, group, K/V).
__global__ __launch_bounds__(256) void append_one_wide_kernel(AppendArgs a) {
  __shared__ float xs[512];
  __shared__ float part[4 * 128];
  if (a.k.lm)
    append_slice_block<true>(a, (int)blockIdx.x, blockIdx.z != 0, (int)blockIdx.y, xs, part);
  else
    append_slice_block<false>(a, (int)blockIdx.x, blockIdx.z != 0, (int)blockIdx.y, xs, part);
}

// Test hook: the quantizer of the multi-token append (min/max codebook: the
// reciprocal fast path with its exact fallback; Lloyd-Max codebook when lm) on
// fp32 rows, canonical packing.
template <int D>
__global__ __launch_bounds__(64) void quantize_rows_kernel(const float* x, float clip, int lm, uint8_t* codes,
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
    GroupQ q;
    if (lm) {
      q = lm_group_wave(v[2 * g], v[2 * g + 1], clip);
      code[2 * g] = lm_code(v[2 * g], q);
      code[2 * g + 1] = lm_code(v[2 * g + 1], q);
    } else {
      const float mx = wave_max(fmaxf(v[2 * g], v[2 * g + 1]));
      const float mn = wave_min(fminf(v[2 * g], v[2 * g + 1]));
      q = group_params(mx, mn, clip);
      const float inv = __builtin_amdgcn_rcpf(q.sf);
      code[2 * g] = quant_code_fast(v[2 * g], q, inv);
      code[2 * g + 1] = quant_code_fast(v[2 * g + 1], q, inv);
    }
    if (lane == 0) meta[row * (D / kGroup) + g] = q.packed;
  }
  store_canonical<PER>(code, lane, [&](int w) { return reinterpret_cast<uint32_t*>(codes + row * (D / 4) + 4 * w); });
}

__global__ __launch_bounds__(256) void set_lens_kernel(SetLensArgs a) {
  const int i = (int)threadIdx.x;
  if (i < a.n) a.lens[a.first + i] = a.vals[i];
}

hipError_t launch_set_lens(const SetLensArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(set_lens_kernel, dim3(1), dim3(kSetLensMax), 0, s, a);
  return hipGetLastError();
}

// Canonical export of the stored K (isv = 0) or V codes: one thread per output byte.
__global__ __launch_bounds__(256) void export_codes_kernel(const uint8_t* stored, uint8_t* canon, int BH,
                                                           int cap, int T, int D, int isv) {
  const size_t nbytes = (size_t)BH * T * (D / 4);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nbytes;
       i += (size_t)gridDim.x * blockDim.x) {
    const int byte = (int)(i % (D / 4));
    const size_t rowi = i / (D / 4);
    const int t = (int)(rowi % T);
    const int bh = (int)(rowi / T);
    if (!isv) {
      canon[i] = stored[kcode_byte(bh, cap, t, byte, D)];
      continue;
    }
    uint32_t out = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int bit;
      const size_t off = vcode_byte(bh, cap, t, 4 * byte + k, D, &bit);
      out |= (uint32_t)((stored[off] >> bit) & 3u) << (2 * k);
    }
    canon[i] = (uint8_t)out;
  }
}

// Plain 16-byte copy used to calibrate bandwidth and traffic counters.
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4* src, uint4* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// Read-only streaming: XOR of every 16-byte word (non-temporal loads, eight in
// flight per thread), one result word per block in out[blockIdx.x] (no atomics:
// thousands of same-address atomics would serialise at the cache).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                          unsigned* out) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  // word-wise XOR into a vector accumulator: four short independent chains,
  // so the arithmetic never holds back the next loads
  u32x4 accv = {0, 0, 0, 0};
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) accv ^= v[u];
  }
  for (; i < n; i += stride) accv ^= src[i];
  unsigned acc = (accv.x ^ accv.y) ^ (accv.z ^ accv.w);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ unsigned wacc[4];
  if ((threadIdx.x & 63) == 0) wacc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (wacc[0] ^ wacc[1]) ^ (wacc[2] ^ wacc[3]);
}

hipError_t launch_stream_read(const void* src, size_t bytes, unsigned* out, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, kStreamReadBlocks);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4*>(src), n, out);
  return hipGetLastError();
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
      hipLaunchKernelGGL(append_one_wide_kernel, dim3((unsigned)(a.batch * a.Hkv), 4, 2), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<512, 1, 8>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* x, int rows, int D, float clip, int lm, uint8_t* codes,
                                uint32_t* meta, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(quantize_rows_kernel<128>, dim3(rows), dim3(64), 0, s, x, clip, lm, codes, meta);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<512>, dim3(rows), dim3(64), 0, s, x, clip, lm, codes, meta);
  return hipGetLastError();
}

hipError_t launch_export_codes(const uint8_t* stored, uint8_t* canon, int BH, int cap, int T, int D, int isv,
                               hipStream_t s) {
  const size_t n = (size_t)BH * T * (D / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(export_codes_kernel, dim3(blocks), dim3(256), 0, s, stored, canon, BH, cap, T, D, isv);
  return hipGetLastError();
}

}  // namespace oscar
