// Launch arguments of the chunked-prefill attention kernel (prefill_attn.hip).
#pragma once

#include "common.h"

namespace oscar {

struct PrefillAttnArgs {
  PlaneDev k, v;
  const uint16_t* q;       // bf16 [B][n][Hq][D]
  void* out;               // [B][n][Hq][D] of out_dtype
  int out_dtype;
  const float* rk;         // fp32 [D][D] of this layer
  const float* rvT;        // fp32 [D][D]: rvT[e][d] = R_V[d][e]
  int absorb_v;
  int B, n, Hq, Hkv, Gq, cap, N, M, T;
  int D;                   // head_dim: 128 or 512
  float scale_log2;        // softmax scale * log2(e)
  const int* lens;         // ragged batch: tokens of sequence b ([B], device); null: every sequence holds T
};

// causal attention of the last n cached positions' queries; returns hipGetLastError()
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s);

}  // namespace oscar
