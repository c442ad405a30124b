// Internal launch interface of the causal attention core (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tps {

constexpr int kAttnHeadDim = 128;  // the one head size the kernel takes
constexpr int kAttnBlock = 128;    // query rows per block: seq_len must be a multiple

struct AttnArgs {
  const void* QKV;     // [tokens][ld_qkv] bf16: Q heads, K heads, V heads of kAttnHeadDim columns each
  void* C;             // [tokens][ld_c] bf16: the query heads' outputs
  int64_t ld_qkv, ld_c;
  int64_t tokens;      // a multiple of seq_len
  int32_t seq_len;     // tokens per sequence (contiguous rows), a multiple of kAttnBlock
  int32_t q_heads, kv_heads;  // q_heads a multiple of kv_heads
  float scale_log2;    // log2(e) / sqrt(head_dim)
};

// Queue the causal attention of every sequence and query head on `stream` (`start`/`stop`: the
// dispatch's own timestamps, for tracing).
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream, hipEvent_t start = nullptr,
                           hipEvent_t stop = nullptr);

}  // namespace tps
