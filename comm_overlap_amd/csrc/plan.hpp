// Host-side plan of the sliced layer shard: validated sizes and slice geometry. No HIP calls here.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tpslice.h"

struct tpslice_plan_s {
  uint32_t magic;
  tpslice_desc_t desc;
  int64_t M, h, Fp, N1, qkv, ctx;  // tokens, hidden, F', up-projection width, QKV width, context width
  int64_t Ms, hc;                  // rows per row slice, hand-off columns per column slice
  // products per row slice of each hand-off output and their width: c pieces of hc columns, or
  // with whole-row hand-off (TPSLICE_F_HANDOFF_ROWS, c > 1) one product of all h columns, since
  // the row slice's copy waits for every column piece anyway
  int32_t pc;
  int64_t pw;
  int32_t r, c, S, E;              // row slices, column slices, worker streams, copy streams
  int32_t qh, kvh;                 // this rank's query / key-value heads
  int32_t trace;                   // tracing enabled
  // k splits (1: none) of the products over all tokens (dW1, dW2, dC, dWo, dWqkv, QKV), of the
  // row slices' up-projection and of the dH groups
  int32_t sp_dw1, sp_dw2, sp_dc, sp_dwo, sp_dwqkv, sp_up, sp_qkv, sp_dh;
  // rows of each weight gradient that its k split covers: its last rows (a tail split, the others
  // unsplit), or 0 for the whole product
  int64_t tl_dw1, tl_dw2, tl_dwo, tl_dwqkv;
  // row slices per dH product: dH runs over groups of gdh consecutive row slices (it is not handed
  // off; each row slice's dX product and hand-off follow it)
  int32_t gdh;
  // row slices per up-projection of the MLP forward (likewise: only the down-projection after it is
  // handed off)
  int32_t gup;
  int32_t tile;                    // tile requested for every product (GemmTile; 0: per product)
  void* rt;                        // device resources (streams, events), created on first execution
};

namespace tps {

constexpr uint32_t kPlanMagic = 0x74707331u;
constexpr uint32_t kDeadMagic = 0xdeadbeefu;
constexpr size_t kWsAlign = 256;
constexpr int kMaxStreams = 8;
constexpr int kMaxCopyStreams = 8;

// Record `fmt` as the calling thread's last error and return `st`.
tpslice_status_t fail(tpslice_status_t st, const char* fmt, ...);
void clear_error();
bool plan_ok(const tpslice_plan_s* p);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace regions (byte offsets) of each operation. Bias gradients are column sums reduced in
// a fixed order through per-chunk partial sums (chunks of kColsumRows token rows, fp32).
constexpr int64_t kColsumRows = 256;
// Split products keep their fp32 partial products in regions of their own (products that may run
// at the same time never share one).
// A split per-slice product has one partial region per worker stream (x_split_bytes each).
struct MlpFwdWs { size_t H, up_split, up_split_bytes, total; };
struct AttnFwdWs { size_t qkv_split, qkv_split_bytes, total; };
struct MlpBwdWs { size_t dU, H, partials, dw1_split, dw2_split, dh_split, dh_split_bytes, total; };
struct AttnBwdWs { size_t partials, dc_split, dwo_split, dwqkv_split, total; };
MlpFwdWs mlp_fwd_ws(const tpslice_plan_s* p);
AttnFwdWs attn_fwd_ws(const tpslice_plan_s* p);
MlpBwdWs mlp_bwd_ws(const tpslice_plan_s* p);
AttnBwdWs attn_bwd_ws(const tpslice_plan_s* p);

}  // namespace tps
