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
  float* lse;          // [tokens][q_heads] fp32: each row's log-sum-exp of its scaled scores (natural
                       // log), or null
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

struct AttnBwdArgs {
  const void* QKV;     // the forward's input [tokens][ld_qkv] bf16
  const void* C;       // the forward's output O [tokens][ld_c] bf16
  const void* dC;      // the gradient of O [tokens][ld_c] bf16
  const float* lse;    // the forward's row log-sum-exp [tokens][q_heads] fp32
  void* dQKV;          // [tokens][ld_qkv] bf16: dQ, dK, dV in QKV's column layout
  float* Dq;           // workspace: [tokens][q_heads] fp32 (filled by launch_attn_bwd)
  float* part;         // workspace: grouped heads' fp32 dK, dV partials (filled by launch_attn_bwd)
  int64_t ld_qkv, ld_c;
  int64_t tokens;
  int32_t seq_len, q_heads, kv_heads;
  float scale;         // 1 / sqrt(head_dim)
  float scale_log2;    // log2(e) / sqrt(head_dim)
};

// Workspace bytes of launch_attn_bwd: D per (token, query head), and when key/value heads serve
// several query heads, fp32 dK and dV partials per query head.
size_t attn_bwd_workspace_bytes(int64_t tokens, int32_t q_heads, int32_t kv_heads);

// Queue the backward pass on `stream`: D, then dK and dV (and the grouped heads' sums), then dQ.
// `ws` (256-byte aligned) holds attn_bwd_workspace_bytes. `start`/`stop` bracket the whole pass.
hipError_t launch_attn_bwd(AttnBwdArgs a, void* ws, hipStream_t stream, hipEvent_t start = nullptr,
                           hipEvent_t stop = nullptr);

}  // namespace tps
