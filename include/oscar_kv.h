/*
 * oscar_kv.h -- C ABI of the OSCAR INT2 KV-cache library for MI355X (gfx950).
 *
 * What it computes (sources are web pages on OSCAR, cited by title/section):
 *  - append: every new post-RoPE K/V vector is rotated by a per-layer
 *    head_dim x head_dim orthogonal matrix ("OSCAR-LLAMACPP-Qwen3-4B-Thinking-
 *    2507-INT2-KV", section "Files", note on the OSCAR rotation; "OSCAR-
 *    RotationZoo", section "File format": one matrix per layer), clipped per
 *    group of 128 along head_dim by a ratio (K 0.96, V 0.92: "OSCAR-RotationZoo",
 *    "How to use", step 2 launch flags), quantized to 2-bit codes with an fp16
 *    scale and zero per group, and packed; the first N and last M positions are
 *    also kept in bf16 (same card, section "Run", env-var table; "OSCAR: 2-bit
 *    KV Cache Quantization for SGLang and llama.cpp", section "What OSCAR
 *    compresses").
 *  - decode attention: one query per sequence attends over the mixed cache,
 *    reading the 2-bit codes directly (fused; the Qwen3-4B card's "Run" table
 *    and the article's section "How the offline rotation is fit"), with the
 *    query rotated by R_K and the output rotated back by R_V^T.
 *
 * Conventions shared by every call:
 *  - vectors are rows: x_rot = x @ R with R row-major fp32 [D][D];
 *  - query head j reads kv head j / (Hq / Hkv);
 *  - a position t of a cache holding T tokens is high precision (bf16) when
 *    t < N or t >= T - M, and INT2 otherwise;
 *  - per group of G values: hi = r*max, lo = r*min, s = (hi - lo)/3 (fp32,
 *    one rounding per op), s16 = fp16(s), z16 = fp16(lo),
 *    c = clamp(rint((x - z16)/s16), 0, 3) (ties to even; c = 0 if s16 == 0);
 *    -0.0 is mapped to +0.0 before the group min/max and before bf16 rounding;
 *  - the canonical 2-bit packing puts code j of a row at byte j/4, bits 2*(j%4).
 *
 * Ownership: the library owns every cache byte (allocated in create, freed in
 * destroy) and private copies of R_K, R_V.  The caller owns q, k, v, out and
 * the stream; device pointers must stay valid until the stream reaches the
 * call.  All calls on one handle must be ordered on one stream (the handle's
 * scratch buffers are shared by its calls); a handle is not thread-safe.
 *
 * Errors: every function returns an oscar_status.  Arguments are validated on
 * the host before anything is enqueued; on an error nothing is enqueued and
 * the cache state is unchanged.  oscar_last_error() returns a thread-local
 * message for the last failure.  Device faults surface at the caller's next
 * synchronisation of the stream.
 */
#ifndef OSCAR_KV_H
#define OSCAR_KV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID_ARG = -1,
  OSCAR_ERR_OUT_OF_MEMORY = -2,
  OSCAR_ERR_CAPACITY = -3,
  OSCAR_ERR_HIP = -4,
  OSCAR_ERR_UNSUPPORTED = -5
} oscar_status;

/* Storage of one of K or V.  BF16 keeps the rotated vector in bf16 at every
 * position (the "--cache-type-v f16" option of the Qwen3-4B card's "Run"
 * section keeps V in high precision). */
typedef enum { OSCAR_KV_INT2 = 0, OSCAR_KV_BF16 = 1 } oscar_kv_dtype;

typedef enum { OSCAR_OUT_F32 = 0, OSCAR_OUT_BF16 = 1, OSCAR_OUT_F16 = 2 } oscar_out_dtype;

/* How a 2-bit code maps to a value of its 128-group ("OSCAR: 2-bit KV Cache
 * Quantization for SGLang and llama.cpp": the Lloyd-Max switch of "Installing
 * OSCAR and running a first Qwen3-8B calibration" and LM_RATIO of "Where OSCAR
 * loses, and the cases it is the wrong tool for").
 *   UNIFORM:    z + s c, z = r min, s = r (max - min) / 3, r the clip ratio;
 *   LLOYD_MAX:  z + s level(c), level = (-1.5104, -0.4528, 0.4528, 1.5104)
 *               (the least-squared-error 4-level quantizer of a unit
 *               Gaussian), z = the group's mean, s = LM_RATIO x its standard
 *               deviation (population: sum of squares / 128); the code is the
 *               nearest level (thresholds 0 and +-0.9816 on (x - z) / s,
 *               ties to the higher code). */
typedef enum { OSCAR_CODEBOOK_UNIFORM = 0, OSCAR_CODEBOOK_LLOYD_MAX = 1 } oscar_codebook;

typedef struct {
  int32_t num_layers;
  int32_t max_batch;        /* sequences per layer                             */
  int32_t num_q_heads;      /* Hq, a multiple of num_kv_heads                   */
  int32_t num_kv_heads;     /* Hkv                                             */
  int32_t head_dim;         /* D: 128 or 512 (a multiple of group_size)        */
  int32_t max_context;      /* capacity per sequence, tokens (>= 1)            */
  int32_t sink_tokens;      /* N: first N positions also kept in bf16 (>= 0)   */
  int32_t recent_tokens;    /* M: last M positions also kept in bf16 (>= 0)    */
  int32_t group_size;       /* G: must be 128                                  */
  float k_clip;             /* clip ratio r for K, in (0, 1]; pages: 0.96      */
  float v_clip;             /* clip ratio r for V, in (0, 1]; pages: 0.92      */
  oscar_kv_dtype k_dtype;
  oscar_kv_dtype v_dtype;
  const float* rot_k;       /* host fp32 [num_layers][D][D], row-major; NULL = identity */
  const float* rot_v;       /* host fp32 [num_layers][D][D], row-major; NULL = identity */
  int32_t device;           /* HIP device ordinal                              */
  int32_t absorb_v_rotation; /* 1: decode attention returns o' = the output in the
                              * V-rotated basis (the caller folds R_V^T into its
                              * output projection: RotationZoo "How to use", the
                              * sglang flag that absorbs the V rotation); 0: o = o' R_V^T */
  int32_t in_quant_hadamard; /* 0: off; 128: the in-quant Hadamard of order 128 (the
                              * quantizer's Hadamard transform of the Qwen3-4B card's
                              * "Run" env-var table; order 128 in the RotationZoo "How to
                              * use" sglang launch).  Both rotations become fp32(R H), H the
                              * orthonormal Sylvester Walsh-Hadamard matrix of order 128 on
                              * each 128-group along head_dim, taken row by row at create
                              * with fast Walsh-Hadamard butterflies in fp64 and rounded
                              * once, so every later step (q rotation, window values, the
                              * quantizer, the V un-rotation by the transpose) is unchanged */
  int32_t codebook;         /* oscar_codebook of both INT2 planes; 0 = UNIFORM       */
  float lm_ratio;           /* LLOYD_MAX only: LM_RATIO in (0, 16]; pages: 1.16.  With
                             * LLOYD_MAX, k_clip and v_clip are not used; decode
                             * attention runs on the general (VALU) kernel and
                             * oscar_prefill_attn returns UNSUPPORTED */
} oscar_kv_config;

typedef struct oscar_kv oscar_kv;

/* Create a cache for cfg on cfg->device (the serving configuration of
 * "OSCAR-RotationZoo", "How to use" step 2: per-layer K and V rotation files,
 * K/V clip ratios, prefix/recent window sizes, int2 cache with quantization
 * group 128; "File format": one head_dim x head_dim matrix per layer).
 * Copies the rotations, allocates
 * every plane for max_batch x max_context tokens per layer and zeroes the
 * metadata.  May synchronise the device (set-up, not the hot path).
 * Errors: INVALID_ARG (bad field, NULL cfg/out), OUT_OF_MEMORY, HIP. */
int oscar_kv_create(const oscar_kv_config* cfg, oscar_kv** out);

/* The append path: each new post-RoPE K/V vector is rotated by its layer's
 * matrix ("OSCAR-LLAMACPP-Qwen3-4B-Thinking-2507-INT2-KV", "Files": the
 * rotation sits in the graph after RoPE), clipped per 128-group by the clip
 * ratio and quantized to 2 bits ("OSCAR-RotationZoo", "How to use" step 2;
 * the article's "How the offline rotation is fit": clipping thresholds bound
 * the values before rounding), with bf16 copies of the first and last
 * positions (Qwen3-4B card, "Run" env-var table).
 * Append n_new tokens to each of sequences 0..batch-1 of `layer`, each at its
 * own length T_b (a ragged batch: the sequences of a layer may hold different
 * numbers of tokens, as the requests of a serving batch do; sequences past
 * `batch` are untouched).
 *   k, v: device bf16 [batch][n_new][Hkv][D], post-RoPE, un-rotated.
 * Per token and kv head: rotate, write the bf16 window copy if the position is
 * in the sink or among the last M positions of its sequence after this append,
 * quantize and pack (INT2 planes) or store bf16 (BF16 planes).  T_b += n_new
 * on success.  The host knows every T_b (it issued every append); for a ragged
 * batch the call first writes the new lengths to a device array of the handle
 * with a small kernel on `stream` (values as kernel arguments: nothing waits).
 * Errors: INVALID_ARG, CAPACITY (some T_b + n_new > max_context), HIP. */
int oscar_kv_append(oscar_kv* kv, int32_t layer, const void* k, const void* v,
                    int32_t batch, int32_t n_new, hipStream_t stream);

/* Decode attention over the mixed INT2 + bf16 cache, read directly by a
 * fused kernel (Qwen3-4B card, "Run": the fused INT2 + f16 flash-attention;
 * the article's "How the offline rotation is fit": no dequantize-then-attend
 * pass), q rotated by R_K so that q k^T is unchanged ("OSCAR-LLAMACPP-Gemma-
 * 4-12B-it-INT2-KV", the rotation paragraph below "Folders"), the output
 * un-rotated by R_V^T ("OSCAR-RotationZoo", "How to use": V is stored
 * rotated, hence the flag that absorbs its rotation).
 * One decode step of attention for `layer`: sequence b of the batch attends
 * over its own T_b cached tokens with the windows of its own length (every
 * sequence of the batch must hold at least one token).
 *   q:   device bf16 [batch][Hq][D], post-RoPE, un-rotated;
 *   out: device [batch][Hq][D] of out_dtype, un-rotated (o = o' @ R_V^T);
 *   softmax_scale <= 0 selects 1/sqrt(D).
 * The INT2 part runs as a split-K flash-decode; the partial results are merged
 * with a log-sum-exp combine that also undoes the V rotation.
 * Errors: INVALID_ARG (including an empty sequence in the batch), HIP. */
int oscar_int2_decode_attn(oscar_kv* kv, int32_t layer, const void* q, void* out,
                           int32_t out_dtype, int32_t batch, float softmax_scale,
                           hipStream_t stream);

/* oscar_int2_decode_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): same arguments, result and errors, and the same kernels, but
 * the call's working memory (the splits' partial results, the q records, the
 * block counters) lives in a file-scope device array of 16 MiB per
 * GPU instead of the handle's buffers.  The call allocates and frees nothing;
 * the array is held by each GPU the library runs on until the process ends,
 * and its counters are cleared once, at the first call on that GPU.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two threads, two handles) race and must be serialised by the
 * caller.  Limit: batch x num_kv_heads <= 65536 and the call's q records,
 * rotated q and batch x num_q_heads x (splits + window blocks) partial slots of
 * (head_dim + 2) floats within 16 MiB less 512 KiB (the 32k, 128k and head_dim
 * 512 benchmark shapes use under 8 MiB).
 * Errors: as oscar_int2_decode_attn, plus CAPACITY (nothing enqueued) when the
 * call's working memory exceeds the array, and HIP if the array's device
 * address cannot be taken. */
int oscar_int2_decode_attn_noalloc(oscar_kv* kv, int32_t layer, const void* q, void* out,
                                   int32_t out_dtype, int32_t batch, float softmax_scale,
                                   hipStream_t stream);

/* One decode step of `layer` as serving runs it (a new token's K/V are
 * cached, then its query attends over every cached token, the new one
 * included; Qwen3-4B card "Run": INT2 cache with the fused flash-attention
 * decode).  Same arguments and errors as oscar_kv_append(k, v, n_new = 1)
 * followed by oscar_int2_decode_attn(q, out), and the stored cache is
 * identical bit for bit; the output is the same attention within the
 * matrix-core kernel's fp16 operand rounding (see below).
 *   k, v: device bf16 [batch][1][Hkv][D]; q, out as in decode_attn.
 * Where the shape has the head_dim 128 matrix-core kernel (4 or 8 query heads
 * per kv head, INT2 K and V) and recent_tokens >= 1: when every block of the
 * attention launch is resident at once and recent_tokens >= 64, one launch
 * does it all (the window block holding the new token appends it; the INT2
 * blocks scale V by the running V-scale maximum from before the token, which
 * the launch then raises), else a short launch appends and writes the q
 * records before the attention launch.  At head_dim 512 (matrix-core path)
 * the append runs in the same launch as the q rotation, before the attention
 * launch.  Other shapes run the two calls' launches in turn. */
int oscar_kv_decode_step(oscar_kv* kv, int32_t layer, const void* k, const void* v, const void* q,
                         void* out, int32_t out_dtype, int32_t batch, float softmax_scale,
                         hipStream_t stream);

/* Chunked-prefill attention over the mixed cache (RotationZoo "How to use":
 * the serving host runs a prefill backend beside the decode one).  The n_q
 * queries are those of the last n_q cached positions of each sequence b of
 * `layer` (normally the chunk just appended): query i, at position
 * p = T_b - n_q + i, attends causally over positions [0, p] of the cache as it
 * stands, i.e. the sink and recent windows of the current length T_b read their
 * bf16 values and every other position its INT2 codes with the group's scale
 * and zero.  q is rotated by R_K; the output is un-rotated by R_V^T (or left in
 * the V-rotated basis with absorb_v_rotation).
 *   q:   device bf16 [batch][n_q][Hq][D], post-RoPE, un-rotated;
 *   out: device [batch][n_q][Hq][D] of out_dtype;
 *   softmax_scale <= 0 selects 1/sqrt(D).
 * head_dim 128 (up to 64 query heads per kv head) or 512 (up to 16), a
 * power-of-two number of query heads per kv head, and the UNIFORM codebook
 * (UNSUPPORTED otherwise).  Nothing is allocated; the cache is read only.
 * Errors: INVALID_ARG (including n_q < 1, n_q > some T_b of the batch),
 * UNSUPPORTED, HIP. */
int oscar_prefill_attn(oscar_kv* kv, int32_t layer, const void* q, void* out, int32_t out_dtype,
                       int32_t batch, int32_t n_q, float softmax_scale, hipStream_t stream);

/* Free every device allocation of the handle (the cache the create call
 * configured).  destroy(NULL) is OK. */
int oscar_kv_destroy(oscar_kv* kv);

/* Thread-local text of the last failure ("" if none). */
const char* oscar_last_error(void);

/* ---- inspection and test hooks (not part of the four-call contract) ---- */

/* Tokens currently held by `layer`: the longest of its sequences (every
 * sequence's count while the batch is uniform). */
int oscar_kv_length(const oscar_kv* kv, int32_t layer, int32_t* tokens);

/* ---- ragged batches: sequences at their own lengths ---- */

/* Append n_new tokens to sequence `seq` alone (the prefill of one request into
 * its slot), at its own length T_seq; the append path of oscar_kv_append.
 *   k, v: device bf16 [n_new][Hkv][D], post-RoPE, un-rotated.
 * Errors: INVALID_ARG (seq outside [0, max_batch), n_new < 1, NULL pointer),
 * CAPACITY (T_seq + n_new > max_context), HIP. */
int oscar_kv_append_seq(oscar_kv* kv, int32_t layer, int32_t seq, const void* k, const void* v,
                        int32_t n_new, hipStream_t stream);

/* Empty sequence `seq` in every layer (a finished request frees its slot);
 * its next tokens start at position 0.  Enqueues a clear of the sequence's
 * running V scale maximum on `stream` (a memset: not for graph capture).
 * Errors: INVALID_ARG, HIP. */
int oscar_kv_reset_seq(oscar_kv* kv, int32_t seq, hipStream_t stream);

/* Tokens held by sequence `seq` of `layer`. */
int oscar_kv_seq_length(const oscar_kv* kv, int32_t layer, int32_t seq, int32_t* tokens);

/* Test switch of the head_dim-128 attention launch's schedule: 3..16 puts
 * every block of a launch on the device at once, with that many blocks per
 * (sequence, kv head) (one INT2 split per block, window chunks carried by
 * some of them); 0 (default) and -1 keep the several-round schedule (INT2
 * splits first, then the window blocks).  Errors: INVALID_ARG. */
int oscar_kv_set_one_round(oscar_kv* kv, int32_t blocks);

/* Device bytes held by the handle. */
int oscar_kv_device_bytes(const oscar_kv* kv, size_t* bytes);

/* Force the number of splits per (sequence, kv head) used by decode attention
 * (INT2 splits of the matrix-core kernel, or all-token splits of the VALU
 * kernel), in [0, 208]; 0 restores the automatic choice.  The count is capped
 * by the number of 64-token tiles.  Errors: INVALID_ARG. */
int oscar_kv_set_num_splits(oscar_kv* kv, int32_t num_splits);

/* Select the decode kernel: 0 = automatic (matrix-core kernels where
 * supported), 1 = the general VALU kernel for every shape.  Test switches of
 * the head_dim-128 matrix-core path: 2 = always a q-record launch before the
 * attention launch, 3 = always one launch whose blocks rotate q themselves
 * (a decode step appends in it when recent_tokens >= 64).  Automatic uses the
 * one launch when all of its blocks are resident at once.  Errors:
 * INVALID_ARG. */
int oscar_kv_set_decode_impl(oscar_kv* kv, int32_t impl);

/* Copy one plane of `layer` to host memory in canonical layout, for all
 * max_batch sequences and the T_l tokens held (synchronises the device).
 *   which: 0 = K, 1 = V.
 *   INT2 plane:  host_codes u8 [max_batch][Hkv][T_l][D/4] (canonical packing),
 *                host_meta  u16 [max_batch][Hkv][T_l][D/G][2] = {s16, z16} bits,
 *                host_sink  u16 [max_batch][Hkv][N][D] bf16 bits,
 *                host_ring  u16 [max_batch][Hkv][M][D] bf16 bits (position t in
 *                slot t % M).
 *   BF16 plane:  host_codes receives u16 [max_batch][Hkv][T_l][D] bf16 bits;
 *                the other pointers are ignored.
 * Any pointer may be NULL to skip that part.  Errors: INVALID_ARG, HIP. */
int oscar_kv_export(oscar_kv* kv, int32_t layer, int32_t which, void* host_codes,
                    void* host_meta, void* host_sink, void* host_ring);

/* As oscar_kv_append, and also write the fp32 rotated vectors (the quantizer
 * inputs) to k_rot / v_rot: device fp32 [batch][n_new][Hkv][D]. */
int oscar_kv_append_dump(oscar_kv* kv, int32_t layer, const void* k, const void* v,
                         int32_t batch, int32_t n_new, float* k_rot, float* v_rot,
                         hipStream_t stream);

/* The append kernel's quantizer on given fp32 rows (no rotation):
 *   x: device fp32 [rows][D]; codes: device u8 [rows][D/4] (canonical packing);
 *   meta: device u16 [rows][D/G][2] = {s16, z16}.
 * Errors: INVALID_ARG (D or G unsupported, NULL pointer, rows < 0), HIP. */
int oscar_quantize_rows(const float* x, int32_t rows, int32_t D, int32_t G, float clip,
                        void* codes, void* meta, hipStream_t stream);

/* The same with the Lloyd-Max codebook and LM_RATIO `ratio` (0 < ratio <= 16):
 * meta = {fp16 s, fp16 mean}. */
int oscar_quantize_rows_lloyd_max(const float* x, int32_t rows, int32_t D, int32_t G, float ratio,
                                  void* codes, void* meta, hipStream_t stream);

/* Kernel timing with HIP events recorded on the caller's stream around the
 * launches of one kernel class: 0 = the INT2 split-K decode kernel, 1 = one
 * whole decode-attention call (q rotation to combine), 2 = append.
 * profile_enable(kv, 1) clears and starts recording (up to 8192 launches per
 * class); profile_read synchronises the recorded events and returns the sum
 * of their durations in milliseconds and the launch count. */
int oscar_kv_profile_enable(oscar_kv* kv, int32_t enable);

/* Calibration kernel for bandwidth and hardware-counter measurements: a plain
 * copy of `bytes` (a multiple of 16) from device buffer src to device buffer
 * dst with 16-byte loads and stores, grid-strided.  Its algorithmic traffic is
 * exactly `bytes` read and `bytes` written.  Errors: INVALID_ARG, HIP. */
int oscar_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Calibration kernel for the achievable HBM read rate: reads `bytes` (a
 * multiple of 16) of device buffer src once, with 16-byte non-temporal loads.
 * xor_out is a device uint32 array of 8192 entries that the caller zeroes;
 * block b of the launch writes entry b, and the XOR of all entries is the XOR
 * of every 32-bit word of src.  Its algorithmic traffic is exactly `bytes`
 * read (plus at most 32 KiB written).  Errors: INVALID_ARG, HIP. */
int oscar_stream_read(const void* src, size_t bytes, void* xor_out, hipStream_t stream);
int oscar_kv_profile_read(oscar_kv* kv, int32_t kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* OSCAR_KV_H */
