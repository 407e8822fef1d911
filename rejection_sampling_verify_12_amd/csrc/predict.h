// Outcome prediction: launchers shared by the stand-alone entry point and the
// fused verification (internal to the library).
#pragma once
#include "topk.h"

namespace sv {

struct PredictArgs {
  const void* draft;          // [B][gamma+1][V] draft logits
  const int32_t* accepted;    // [B] or NULL (candidates only)
  const int32_t* out_tokens;  // [B][gamma+1] or NULL
  int32_t* cand;              // [B][gamma+1][3]
  int32_t* hit;               // [B] or NULL
  int32_t* cand_idx;          // [B] or NULL
  Top3* part;                 // [B][gamma+1][nc] chunk records
  int B, gamma, V, nc, chunk;
};

// Bytes of chunk records for chunks of kChunk logits.
size_t predict_part_bytes(int B, int gamma, int V);

// Stand-alone: rank every draft row chunk by chunk (element keys in `part`),
// then merge and evaluate the hit.
hipError_t predict_launch_rows(const PredictArgs& a, int dtype, bool vec, hipStream_t st);

// From lane leaders that the verification's stream items left in `part`
// (chunks of a.chunk logits): re-read the leading lanes, rank, evaluate.
hipError_t predict_launch_leaders(const PredictArgs& a, int dtype, hipStream_t st);

}  // namespace sv
