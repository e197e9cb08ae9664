// Internal definitions shared by the host library and the gfx950 kernels:
// storage layout of the cache planes, number-format helpers, launcher
// declarations.  Nothing here is part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kGroup = 128;           // quantization group along head_dim
constexpr int kTile = 64;             // tokens per decode tile / V storage block
constexpr int kMaxSplits = 256;       // partial-result slots per (sequence, head)
constexpr int kQPub = 4 * 128 + 8 + 1024;  // published q of 4 query heads: fp32 q, sums, exponents,
                                           // two-piece fp16 operands in two instruction layouts
constexpr int kMaxGq = 16;            // query heads per kv head handled by the VALU kernel
constexpr int kMaxOneRound = 16;      // INT2 splits per (sequence, kv head) of a one-round launch

// ---------------------------------------------------------------------------
// Storage layout (per layer; b = sequence, h = kv head, t = position, d = dim)
//
//  K INT2 codes : canonical packing within a token row (code d at byte d/4,
//                 bits 2*(d%4)), rows stored by 64-token tile in 16-byte
//                 chunks: byte i of token t sits in chunk i/16 of the tile,
//                 and a chunk holds that 16-byte piece of the tile's 64 rows
//                 (token t%64 at 16*(t%64)).  A decode lane owns one token
//                 row and each of its 16-byte loads is contiguous across the
//                 wave.
//  K/V meta     : u32 [B][Hkv][D/128][cap] = fp16 scale (low) | fp16 zero (high);
//                 group-major, so the scales of one 128-wide group are
//                 contiguous over tokens
//  V INT2 codes : tiled for the PV matrix-core operand.  For every 64-token
//                 block and every 128-wide slice of head_dim there is a 2 KiB
//                 tile of 64 lane records of 32 bytes, stored as two 1 KiB
//                 halves (bytes 0-15 of every record, then bytes 16-31), so
//                 each 16-byte load is contiguous across the wave.  Within a slice,
//                 dim ds = d % 128 belongs to lane 4*((ds%64)/4) + ds%4 and to
//                 half hh = ds/64; token tb = t % 64 lives in 32-bit word tb/8
//                 of that record at bit
//                   16*(tb%2) + 8*hh + 2*(2*((tb/4)%2) + (tb/2)%2).
//                 One AND mask of a word yields two fp16 operands (tokens tb,
//                 tb^1) scaled by a power of four that depends only on (tb/2)%4.
//  sink / ring  : bf16 [B][Hkv][N][D] and [B][Hkv][M][D]; position t of the
//                 recent window lives in ring slot t % M.
//  BF16 plane   : bf16 [B][Hkv][cap][D] for every position.
//  V scale max  : f32 [B][Hkv], running max of stored V scales (the decode
//                 kernel sizes its fp16 operand range from it).
// cap is max_context rounded up to a multiple of 64.
// ---------------------------------------------------------------------------

// byte offset of byte i (0 <= i < D/4) of token t's K code row
__host__ __device__ inline size_t kcode_byte(int bh, int cap, int t, int i, int D) {
  const size_t tile = (size_t)bh * (cap / kTile) + (t >> 6);
  return tile * (size_t)(kTile * D / 4) + (size_t)(i >> 4) * 1024 + (size_t)(t & 63) * 16 + (i & 15);
}

// index of the scale|zero word of group g of token t
__host__ __device__ inline size_t meta_index(int bh, int cap, int t, int g, int D) {
  return ((size_t)bh * (D / kGroup) + g) * (size_t)cap + t;
}

// byte offset and bit of the 2-bit V code (t, d) in the tiled layout
__host__ __device__ inline size_t vcode_byte(int bh, int cap, int t, int d, int D, int* bit) {
  const int tb = t & 63, ds = d & 127, slice = d >> 7;
  const int hh = ds >> 6;
  const int lane = 4 * ((ds & 63) >> 2) + (ds & 3);
  const int bitpos = 16 * (tb & 1) + 8 * hh + 2 * (2 * ((tb >> 2) & 1) + ((tb >> 1) & 1));
  *bit = bitpos & 7;
  const size_t tile = ((size_t)bh * (cap / kTile) + (t >> 6)) * (size_t)(D / 128) + slice;
  const int rec = (tb >> 3) * 4 + (bitpos >> 3);     // byte of the lane record, 0..31
  return tile * 2048 + (size_t)(rec >> 4) * 1024 + (size_t)lane * 16 + (rec & 15);
}

// first byte of the 2 KiB V code tile of the 64-token tile holding t and slice g
__host__ __device__ inline size_t vcode_tile_base(int bh, int cap, int t, int g, int D) {
  return (((size_t)bh * (cap / kTile) + (t >> 6)) * (size_t)(D / 128) + g) * 2048;
}

__host__ __device__ inline size_t row_offset(int bh, int rows, int t, int D) {
  return ((size_t)bh * rows + t) * (size_t)D;
}

// s_waitcnt operand (gfx9 encoding) that waits for lgkmcnt = 0 only (vmcnt and
// expcnt at their maxima).
constexpr int kWaitLds = 0xc07f;

// Lanes of one wave exchange values through shared memory: every lane's
// earlier shared-memory writes are complete and visible to every lane's later
// reads.  The wavefront-scope release and acquire fences order the accesses in
// the language's memory model and keep the compiler from moving them across
// (at that scope they emit no instruction); the wait completes the wave's own
// writes, which the hardware then serves in order.  A fence of wider scope
// would also wait for every vector memory load in flight (the next tiles),
// which these loops keep outstanding.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(kWaitLds);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return v.f;
}

// float32 -> bf16, round to nearest even (finite inputs)
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  const uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook: the 4-level quantizer of least mean squared error for a
// unit Gaussian (Max's table: levels +-0.4528 and +-1.5104, decision
// thresholds 0 and +-0.9816, the midpoints of neighbouring levels), placed on
// a group's mean with the step s = LM_RATIO x the group's standard deviation
// ("OSCAR: 2-bit KV Cache Quantization for SGLang and llama.cpp": the
// Lloyd-Max switch in "Installing OSCAR and running a first Qwen3-8B
// calibration", LM_RATIO = 1.16 in "Where OSCAR loses").  Code c stands for
// z + s * level(c); the scale|zero word holds fp16 s and fp16 mean.
// ---------------------------------------------------------------------------
constexpr float kLmLevel0 = -1.5104f, kLmLevel1 = -0.4528f, kLmLevel2 = 0.4528f, kLmLevel3 = 1.5104f;
constexpr float kLmThreshold = 0.9816f;

__host__ __device__ inline float lm_level(uint32_t c) {
  const float lo = (c & 1u) ? kLmLevel1 : kLmLevel0;
  const float hi = (c & 1u) ? kLmLevel3 : kLmLevel2;
  return (c & 2u) ? hi : lo;
}

// ---------------------------------------------------------------------------
// launch arguments
// ---------------------------------------------------------------------------

struct PlaneDev {
  uint8_t* codes;     // INT2 codes (K canonical or V tiled); null for BF16 planes
  uint32_t* meta;     // fp16 scale | fp16 zero per group
  uint16_t* sink;     // bf16 [B][Hkv][N][D]
  uint16_t* ring;     // bf16 [B][Hkv][M][D]
  uint16_t* full;     // bf16 [B][Hkv][cap][D]; BF16 planes only
  float* smax;        // [B][Hkv] running max of stored scales (V only)
  float clip;         // clip ratio (min/max codebook) or LM_RATIO (Lloyd-Max codebook)
  int is_bf16;
  int tiled;          // 1 for the V code layout
  int lm;             // 1: Lloyd-Max codebook (code c = z + s * lm_level(c)); 0: z + s * c
};

struct AppendArgs {
  PlaneDev k, v;
  const uint16_t* kin;    // bf16 [batch][n_new][Hkv][D]
  const uint16_t* vin;
  const float* rk;        // fp32 [D][D] for this layer
  const float* rv;
  const uint16_t* rk3;    // bf16 [3][D][D]: R_K^T as three pieces summing to it (matrix-core prefill)
  const uint16_t* rv3;
  float* kdump;           // optional fp32 [batch][n_new][Hkv][D]
  float* vdump;
  int batch, n_new, Hkv, D, cap, N, M, T_old, T_new;
  const int* lens;        // ragged batch: tokens of sequence b after this append ([batch], device);
                          // null: every sequence goes from T_old to T_new
};

// Token counts of sequence b around an append: [T_old, T_new).
__device__ inline int2 append_range(const AppendArgs& a, int b) {
  if (!a.lens) return make_int2(a.T_old, a.T_new);
  const int t1 = a.lens[b];
  return make_int2(t1 - a.n_new, t1);
}

struct QRotArgs {
  const uint16_t* q;      // bf16 [B][Hq][D]
  const float* rk;        // fp32 [D][D]
  float* qrot;            // fp32 [B][Hq][D], q @ R_K * scale * log2(e)
  int B, Hq, Hkv, D;
  float scale_log2;
};

struct SegPlan {           // up to two token segments, split into `splits` chunks
  int a0, b0, a1, b1;      // [a0, b0) then [a1, b1) (either may be empty)
  int splits;              // blocks along y
  int chunk;               // tokens of the concatenated segments per split (multiple of 64)
  int slot0;               // first partial slot written by split 0
};

struct CombineArgs {
  const float* partials;
  const float* rvT;        // fp32 [D][D]: rvT[e][d] = R_V[d][e]
  void* out;
  int out_dtype;
  int B, Hq, Hkv, D, nslots;
  int pstride;             // partial slots per (sequence, query head) in `partials` (>= nslots)
  int absorb_v;            // 1: write the merged o' (V-rotated basis), no un-rotation
};

struct DecodeArgs {
  PlaneDev k, v;
  const float* qrot;       // rotated q of the general kernel
  float* qpub;             // [B*Hkv*G][kQPub]: rotated q of each head group, written by the
                           // prologue launch before an attention launch that does not rotate
                           // q itself (head_dim 128), or by the q rotation launch (512)
  float* partials;         // [B][Hq][pstride][D+2]
  int pstride;             // partial slots per (sequence, query head)
  int Hq, Hkv, D, cap, N, M, T;
  int Gq, G;               // query heads per kv head; head groups of 4 (matrix-core kernel)
  SegPlan plan;            // INT2 range (matrix-core kernel) or all tokens (VALU kernel)
  SegPlan win;             // bf16 window segments handled by extra blocks of the
                           // matrix-core launch (win.splits blocks of <= 64 tokens)
  unsigned* counters;      // [B*Hkv] finished blocks per (sequence, kv head); every
                           // entry is zero between launches (the last block resets it)
  CombineArgs comb;        // merge done by the last block of each (sequence, kv head)
  const uint16_t* q;       // bf16 [B][Hq][D] (matrix-core launch rotates q itself)
  const float* rk;         // fp32 [D][D] of this layer
  float scale_log2;        // softmax scale * log2(e)
  int app_blocks;          // 2 when the launch also appends this step's token, else 0; a
                           // self-rotating head_dim-128 launch then points app.v.smax at a
                           // per-(sequence, kv head) pending slot (zero between launches)
  int self_rotate;         // head_dim 128: 1 = the attention launch is the whole call (every
                           // block rotates its q; the window block holding a step's token
                           // appends it); 0 = decode_prologue_kernel ran first
  int int2_lead;           // INT2 splits dispatched before the window blocks
  int win_blocks;          // window blocks of the launch (win.splits)
  int one_round;           // 1: one block per INT2 split and nothing else, every block resident at
                           // once; window chunks and the append are extra work of some splits
  float share[kMaxOneRound + 1];   // one_round: INT2 tiles of splits [0, s) = share[s] x the range's tiles
  int ring0;               // ring slot of the first recent token win.a1 (win.a1 % M)
  AppendArgs app;          // that append (n_new = 1); T above counts the new token
  const int* lens;         // ragged batch: tokens of sequence b ([B], device, this launch's appended
                           // token included); null: every sequence holds T.  With lens, T, plan and
                           // win describe the longest sequence (grid and chunk sizes) and every
                           // block derives its sequence's own token sets
};

// launchers (defined in the .hip files); return hipGetLastError()
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_prefill(const AppendArgs& a, hipStream_t s);   // n_new > 1, rotation on matrix cores
hipError_t launch_quantize_rows(const float* x, int rows, int D, float clip, int lm, uint8_t* codes,
                                uint32_t* meta, hipStream_t s);
hipError_t launch_qrot(const QRotArgs& a, hipStream_t s);
hipError_t launch_decode_valu(const DecodeArgs& a, int B, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int waves_per_block, hipStream_t s);
hipError_t launch_decode_prologue(const DecodeArgs& a, int B, hipStream_t s);  // head_dim 128: q records
                                                                               // (and the step's append)
int decode_mfma_resident_blocks(int device, int G);   // blocks of the matrix-core kernel resident at once
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_wide_qrot(const DecodeArgs& a, int B, hipStream_t s);     // head_dim 512: rotated q records
                                                                            // (and the step's append when a.app_blocks)
hipError_t launch_decode_wide(const DecodeArgs& a, int B, hipStream_t s);   // head_dim 512: INT2 + window partials
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
constexpr int kStreamReadBlocks = 8192;   // result words of the read calibration kernel
hipError_t launch_stream_read(const void* src, size_t bytes, unsigned* out, hipStream_t s);
// Working memory of the allocation-free decode call: a file-scope device array
// of kStaticScratchBytes per GPU (scratch.hip).  static_scratch returns this
// device's address of it (clearing its counter region on first use, on
// `stream`).
constexpr size_t kStaticScratchBytes = 16u << 20;
constexpr size_t kCounterBytes = 256u << 10;          // 65536 (sequence, kv head) pairs
hipError_t static_scratch(int device, hipStream_t stream, unsigned char** ptr);
// lens[first + i] = vals[i], i < n (n <= kSetLensMax): per-sequence token
// counts written in stream order, the values travelling as kernel arguments
constexpr int kSetLensMax = 256;
struct SetLensArgs {
  int* lens;
  int first, n;
  int vals[kSetLensMax];
};
hipError_t launch_set_lens(const SetLensArgs& a, hipStream_t s);
hipError_t launch_export_codes(const uint8_t* stored, uint8_t* canon, int BH, int cap, int T, int D, int isv,
                               hipStream_t s);

}  // namespace oscar
