// Plan construction and validation (host only, no HIP calls): sizes of one rank's share and the
// geometry of its independent pieces (Domino page, Abstract: one batch broken into independent
// pieces). Rows: r equal contiguous token ranges. Columns: c equal ranges of the hand-off output.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "plan.hpp"
#include "attn.hpp"
#include "gemm.hpp"

namespace tps {

static thread_local char g_last_error[512] = "";

tpslice_status_t fail(tpslice_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

bool plan_ok(const tpslice_plan_s* p) { return p != nullptr && p->magic == kPlanMagic; }

static int32_t worker_regions(const tpslice_plan_s* p) { return p->S > 0 ? p->S : 1; }

MlpFwdWs mlp_fwd_ws(const tpslice_plan_s* p) {
  MlpFwdWs w{};
  w.H = 0;
  w.up_split = align_up(size_t(p->M) * size_t(p->Fp) * 2, kWsAlign);
  w.up_split_bytes = align_up(split_partials_bytes(p->Ms * p->gup, p->N1, p->sp_up), kWsAlign);
  w.total = w.up_split + w.up_split_bytes * size_t(worker_regions(p));
  return w;
}

AttnFwdWs attn_fwd_ws(const tpslice_plan_s* p) {
  AttnFwdWs w{};
  w.qkv_split = 0;  // QKV runs over all tokens: one partials region
  w.qkv_split_bytes = align_up(split_partials_bytes(p->M, p->qkv, p->sp_qkv), kWsAlign);
  w.total = w.qkv_split_bytes;
  return w;
}

static size_t partials_bytes(int64_t M, int64_t N) {
  return size_t((M + kColsumRows - 1) / kColsumRows) * size_t(N) * sizeof(float);
}

MlpBwdWs mlp_bwd_ws(const tpslice_plan_s* p) {
  MlpBwdWs w{};
  w.dU = 0;
  w.H = align_up(size_t(p->M) * size_t(p->N1) * 2, kWsAlign);
  w.partials = w.H + align_up(size_t(p->M) * size_t(p->Fp) * 2, kWsAlign);
  w.dw1_split = w.partials + align_up(partials_bytes(p->M, p->N1), kWsAlign);
  w.dw2_split = w.dw1_split + align_up(split_partials_bytes(p->tl_dw1 ? p->tl_dw1 : p->N1, p->h, p->sp_dw1), kWsAlign);
  w.dh_split = w.dw2_split + align_up(split_partials_bytes(p->tl_dw2 ? p->tl_dw2 : p->h, p->Fp, p->sp_dw2), kWsAlign);
  w.dh_split_bytes = align_up(split_partials_bytes(p->Ms * p->gdh, p->Fp, p->sp_dh), kWsAlign);
  w.total = w.dh_split + w.dh_split_bytes * size_t(worker_regions(p));
  return w;
}

AttnBwdWs attn_bwd_ws(const tpslice_plan_s* p) {
  AttnBwdWs w{};
  w.partials = 0;
  w.dc_split = align_up(partials_bytes(p->M, p->qkv), kWsAlign);
  w.dwo_split = w.dc_split + align_up(split_partials_bytes(p->M, p->ctx, p->sp_dc), kWsAlign);
  w.dwqkv_split = w.dwo_split + align_up(split_partials_bytes(p->tl_dwo ? p->tl_dwo : p->h, p->ctx, p->sp_dwo), kWsAlign);
  w.total = w.dwqkv_split +
            align_up(split_partials_bytes(p->tl_dwqkv ? p->tl_dwqkv : p->qkv, p->h, p->sp_dwqkv), kWsAlign);
  return w;
}

}  // namespace tps

using namespace tps;

static bool fits_4g(int64_t rows, int64_t cols, int64_t elem) {
  // every operand is addressed through 32-bit buffer offsets
  const double bytes = double(rows) * double(cols) * double(elem);
  return rows >= 0 && cols >= 0 && bytes < 4294967296.0 - 4096.0;
}

// Row slices per product of a producer that is not handed off (the up-projection, dH): the fewest
// (a power of two dividing r) whose product over that many row slices, with `splits` k splits,
// comes within 5% of the best estimated time per row slice.
static int32_t slice_group(int32_t r, int64_t Ms, int64_t N, int64_t K, int layout, int epi, int splits) {
  if (Ms <= 0) return 1;
  double per[6] = {0}, best = 1e300;
  int n = 0;
  for (int g = 1; g <= r && n < 6; g *= 2, ++n) {
    per[n] = r % g ? 1e300 : estimate_product_us(Ms * g, N, K, layout, epi, true, splits) / g;
    best = std::min(best, per[n]);
  }
  for (int k = 0, g = 1; k < n; ++k, g *= 2)
    if (per[k] <= best * 1.05) return g;
  return 1;
}

// Worker streams when the descriptor leaves them open. For an MLP shard (no attention heads): the
// share of a row slice's forward product work that leaves compute units idle, each product's flops
// times the share of its rounds of blocks it leaves empty on the 256 CUs (with the tile it takes
// alone; a product split along k counts the blocks of its 256 x 256 partial products). One stream
// (slices in order) when that share is at most 5%; otherwise two, so that each slice's products
// share the CUs with the next slice's first product (the schedule choice between finer pieces and
// more overlap, by the products' static sizes: FiCCO page, Abstract). A layer shard (attention
// heads) takes one stream: its QKV projection, dC and every weight gradient run over all tokens on
// worker 0 and dH over groups of row slices, so only the hand-off products could share the CUs,
// and a second stream's event hops cost more than that gains. So does a shard whose up-projection
// runs over groups of row slices. Measured with 2048-row slices: the Llama-2 7B MLP (its
// up-projection per row slice fills 200 of 256 CUs: 31% idle work) 914 TFLOP/s with one stream
// against 972 with two, and 971 with one stream and the up-projection over all four row slices
// (668 with two: each row slice's down-projection then waits for the one before on the other
// stream); the Llama-2 13B layer 802 with one against 709 with two; the Llama-3 70B layer 1130
// against 1140, within run-to-run spread.
static int32_t default_streams(const tpslice_plan_s* p) {
  constexpr int64_t kCUs = 256;
  // (an up-projection over groups of row slices fills the GPU by itself and leaves each row slice
  // one product, the down-projection: two streams would only order those across streams)
  if (p->r <= 1 || p->qh > 0 || p->gup > 1) return 1;
  const bool glu = p->desc.act == TPSLICE_ACT_SWIGLU;
  const int64_t h = p->desc.hidden;
  struct P { int64_t rows, n, k; int epi; int splits; double flops; };
  const P prods[] = {
      {p->Ms * p->gup, p->Fp, h, glu ? kEpiSwiglu : kEpiGelu, p->sp_up, double(p->N1) * double(h)},
      {p->Ms, p->pw, p->Fp, kEpiBf16, 1, double(h) * double(p->Fp)},
  };
  double idle = 0.0, total = 0.0;
  for (const P& q : prods) {
    if (q.n <= 0 || q.k <= 0) continue;
    double fill = 0.0;
    if (q.splits > 1) {
      const int64_t nt = q.epi == kEpiSwiglu ? 2 * q.n : q.n;  // both halves: the split partials' width
      const int64_t blocks = ((q.rows + 255) / 256) * ((nt + 255) / 256) * q.splits;
      const int64_t rounds = (blocks + kCUs - 1) / kCUs;
      fill = double(blocks) / double(rounds * kCUs);
    } else {
      choose_tile(q.rows, q.n, q.k, kFwd, q.epi, true, &fill);
    }
    idle += q.flops * (1.0 - fill);
    total += q.flops;
  }
  return total > 0.0 && idle > 0.05 * total ? 2 : 1;
}

// The forward schedule of a plan whose geometry (r, c, Ms, pc, pw) is set: the up-projection's k
// split (the whole batch's), its row-slice group and the worker streams. Two worker streams and
// grouped up-projections exclude each other: with two streams each row slice's up-projection fills
// the CUs the other stream's products leave idle; grouped, it fills them by itself, and the row
// slices are left one product each.
static void forward_schedule(tpslice_plan_s* q) {
  const tpslice_desc_t* d = &q->desc;
  const int epi_up = d->act == TPSLICE_ACT_SWIGLU ? kEpiSwiglu : kEpiGelu;
  q->sp_up = choose_split(d->tokens, q->N1, d->hidden);
  const bool forced = d->up_group > 0 && q->r % d->up_group == 0;
  q->gup = forced ? d->up_group : 1;
  if (d->flags & TPSLICE_F_SERIALIZE) q->S = 1;
  else if (d->n_streams > 0) q->S = d->n_streams;
  else q->S = default_streams(q);
  if (!forced && q->S == 1) q->gup = slice_group(q->r, q->Ms, q->Fp, d->hidden, kFwd, epi_up, q->sp_up);
}

// Rate of this GPU's local hand-off copy for large pieces (DMA engine, measured 550-760 GB/s for
// 40-70 MB copies) and the fixed cost of one copy.
constexpr double kLocalHandoffGbps = 600.0;
constexpr double kCopyFixedUs = 20.0;
// Pipelined plans close each row slice's copies with a fence and an event that the next call
// waits for: measured about 20 us per row slice with one worker stream and 80 us with two (the
// copy stream then also waits for events of alternating workers).
constexpr double kSliceSyncUs1 = 20.0, kSliceSyncUs2 = 80.0;

// Predicted time (us) of one call of the forward products with r row and c column slices: the
// per-slice products from the GEMM cost model, the hand-off pieces at `gbps` plus a fixed cost per
// copy. With two worker streams, adjacent row slices run side by side, which the model takes as
// one product over twice the rows for each pair. Row slice i's copies run while later slices
// compute, the last ones under the QKV projection over all tokens (which follows the slices).
static double predict_forward_us(const tpslice_desc_t* d, int64_t Fp, int64_t N1, int64_t qkv, int64_t ctx, int r,
                                 int c, int S, int gup, double gbps) {
  const int64_t M = d->tokens, Ms = M / r, h = d->hidden;
  const int pc = (c > 1 && (d->flags & TPSLICE_F_HANDOFF_ROWS)) ? 1 : c;  // products per row slice
  const int64_t pw = h / pc;
  const int pair = (S > 1 && r > 1) ? 2 : 1;
  const int64_t Mp = Ms * pair;  // rows of the products that share the GPU at once
  const bool alone = pair == 1;
  const int epi_up = d->act == TPSLICE_ACT_SWIGLU ? kEpiSwiglu : kEpiGelu;
  // the up-projection over groups of row slices (see tpslice_plan), its time shared by the group
  const int sp_up = choose_split(M, N1, h);
  const double up_us = gup > 1 ? pair * estimate_product_us(Ms * gup, Fp, h, kFwd, epi_up, true, sp_up) / gup
                               : estimate_product_us(Mp, Fp, h, kFwd, epi_up, alone, sp_up);
  double group_us = up_us + pc * estimate_product_us(Mp, pw, Fp, kFwd, kEpiBf16, alone);
  int tensors = 1;
  double tail_us = 0.0;  // products over all tokens after the slices
  if (qkv > 0) {
    group_us += pc * estimate_product_us(Mp, pw, ctx, kFwd, kEpiBf16, alone);
    const int s = choose_split(M, qkv, h);
    tail_us = std::min(estimate_product_us(M, qkv, h, kFwd, kEpiBf16, true, s),
                       estimate_product_us(M, qkv, h, kFwd, kEpiBf16, true, 1));
    tensors = 2;
  }
  const double sliced_us = group_us * double((r + pair - 1) / pair);
  const double slice_us = sliced_us / r;
  // one row slice's copies: c pieces, or one whole-row copy (the same bytes, one fixed cost)
  const double copy_us = double(Ms) * double(h) * 2.0 * tensors / (gbps * 1e3) + pc * kCopyFixedUs * tensors;
  // Pipelined: the next call's row slice 0 waits for this call's copy of row slice 0, which the rest
  // of this call (its later slices and the all-token products) covers only in part; with one row
  // slice nothing covers it.
  if (d->flags & TPSLICE_F_PIPELINE) {
    const double exposed = std::max(0.0, copy_us - (sliced_us - slice_us + tail_us));
    return std::max(sliced_us + tail_us, r * (copy_us + (S > 1 ? kSliceSyncUs2 : kSliceSyncUs1))) + exposed;
  }
  return std::max({sliced_us + tail_us, sliced_us + copy_us, slice_us + r * copy_us});
}

// Slice counts for a descriptor with r or c = 0 (the header describes the rule).
static void choose_slices(const tpslice_desc_t* d, int64_t Fp, int64_t N1, int64_t qkv, int64_t ctx, int32_t* r_out,
                          int32_t* c_out) {
  const double gbps = d->handoff_gbps > 0.0f ? double(d->handoff_gbps) : kLocalHandoffGbps;
  int32_t best_r = d->n_row_slices > 0 ? d->n_row_slices : 1;
  int32_t best_c = d->n_col_slices > 0 ? d->n_col_slices : 1;
  if (d->tokens <= 0) {
    *r_out = best_r;
    *c_out = best_c;
    return;
  }
  double best = 1e300;
  int best_pieces = 0;
  for (int32_t r : {1, 2, 4, 8, 16}) {
    if (d->n_row_slices > 0 && r != d->n_row_slices) continue;
    if (d->tokens % r) continue;
    for (int32_t c : {1, 2, 4}) {
      if (d->n_col_slices > 0 && c != d->n_col_slices) continue;
      if (d->hidden % c || (d->hidden / c) % 8) continue;
      // the worker streams the plan would take for this slicing
      tpslice_plan_s q{};
      q.desc = *d;
      q.Fp = Fp; q.N1 = N1; q.qkv = qkv; q.ctx = ctx; q.qh = qkv > 0 ? 1 : 0;
      q.r = r; q.c = c; q.Ms = d->tokens / r; q.hc = d->hidden / c;
      q.pc = (c > 1 && (d->flags & TPSLICE_F_HANDOFF_ROWS)) ? 1 : c;
      q.pw = d->hidden / q.pc;
      forward_schedule(&q);
      const double t = predict_forward_us(d, Fp, N1, qkv, ctx, r, c, q.S, q.gup, gbps);
      const int pieces = r * c;
      // candidates with more pieces must be 2% faster to be taken
      const bool better = pieces <= best_pieces ? t < best : t < best * 0.98;
      if (best_pieces == 0 || better) {
        best = t;
        best_pieces = pieces;
        best_r = r;
        best_c = c;
      }
    }
  }
  *r_out = best_r;
  *c_out = best_c;
}

extern "C" tpslice_status_t tpslice_plan(const tpslice_desc_t* d, tpslice_plan_t* out) {
  clear_error();
  if (!out) return fail(TPSLICE_ERR_INVALID, "tpslice_plan: out is NULL");
  *out = nullptr;
  if (!d) return fail(TPSLICE_ERR_INVALID, "tpslice_plan: desc is NULL");
  if (d->act != TPSLICE_ACT_GELU && d->act != TPSLICE_ACT_SWIGLU)
    return fail(TPSLICE_ERR_INVALID, "act %d is not TPSLICE_ACT_GELU or TPSLICE_ACT_SWIGLU", d->act);
  if (d->flags &
      ~(TPSLICE_F_SERIALIZE | TPSLICE_F_COPY_BLIT | TPSLICE_F_PIPELINE | TPSLICE_F_HANDOFF_ROWS |
        TPSLICE_F_CALLER_WORKER | TPSLICE_F_TILE_MASK))
    return fail(TPSLICE_ERR_INVALID, "unknown flag bits 0x%x", d->flags);
  if (((d->flags & TPSLICE_F_TILE_MASK) >> TPSLICE_F_TILE_SHIFT) >= TPSLICE_TILE_COUNT)
    return fail(TPSLICE_ERR_INVALID, "tile id %u in the flags is not one of 0..%d",
                (d->flags & TPSLICE_F_TILE_MASK) >> TPSLICE_F_TILE_SHIFT, TPSLICE_TILE_COUNT - 1);
  if (d->tokens < 0) return fail(TPSLICE_ERR_SHAPE, "tokens %lld < 0", (long long)d->tokens);
  if (d->hidden <= 0 || d->hidden % 8)
    return fail(TPSLICE_ERR_SHAPE, "hidden %lld must be a positive multiple of 8", (long long)d->hidden);
  if (d->tp_size < 1) return fail(TPSLICE_ERR_SHAPE, "tp_size %d < 1", d->tp_size);
  if (d->ffn <= 0 || d->ffn % d->tp_size)
    return fail(TPSLICE_ERR_SHAPE, "ffn %lld is not a positive multiple of tp_size %d", (long long)d->ffn,
                d->tp_size);
  const int64_t Fp = d->ffn / d->tp_size;
  if (Fp % 8) return fail(TPSLICE_ERR_SHAPE, "ffn shard %lld is not a multiple of 8", (long long)Fp);
  if (d->n_row_slices < 0 || d->n_col_slices < 0)
    return fail(TPSLICE_ERR_SHAPE, "slice counts r=%d c=%d must be >= 0 (0: automatic)", d->n_row_slices,
                d->n_col_slices);
  if (!(d->handoff_gbps >= 0.0f) || d->handoff_gbps > 1e6f)
    return fail(TPSLICE_ERR_SHAPE, "handoff_gbps %g outside [0, 1e6]", double(d->handoff_gbps));
  if (d->n_row_slices > 0 && d->tokens % d->n_row_slices)
    return fail(TPSLICE_ERR_SHAPE, "%d row slices do not divide %lld tokens evenly", d->n_row_slices,
                (long long)d->tokens);
  if (d->n_col_slices > 0 && (d->hidden % d->n_col_slices || (d->hidden / d->n_col_slices) % 8))
    return fail(TPSLICE_ERR_SHAPE, "%d column slices of hidden %lld must be equal multiples of 8",
                d->n_col_slices, (long long)d->hidden);
  if (d->dh_group < 0 || (d->dh_group & (d->dh_group - 1)) != 0 || d->up_group < 0 ||
      (d->up_group & (d->up_group - 1)) != 0)
    return fail(TPSLICE_ERR_INVALID, "up_group %d and dh_group %d must be 0 or powers of two", d->up_group,
                d->dh_group);
  if (d->n_streams < 0 || d->n_streams > kMaxStreams)
    return fail(TPSLICE_ERR_SHAPE, "n_streams %d outside [0, %d]", d->n_streams, kMaxStreams);
  if (d->n_copy_streams < 0 || d->n_copy_streams > kMaxCopyStreams)
    return fail(TPSLICE_ERR_SHAPE, "n_copy_streams %d outside [0, %d]", d->n_copy_streams, kMaxCopyStreams);
  int32_t qh = 0, kvh = 0;
  if (d->n_heads < 0 || d->n_kv_heads < 0 || d->head_dim < 0)
    return fail(TPSLICE_ERR_SHAPE, "negative head counts");
  if (d->n_heads > 0) {
    if (d->head_dim <= 0 || d->head_dim % 8)
      return fail(TPSLICE_ERR_SHAPE, "head_dim %d must be a positive multiple of 8", d->head_dim);
    if (d->n_heads % d->tp_size)
      return fail(TPSLICE_ERR_SHAPE, "%d heads do not split over tp_size %d", d->n_heads, d->tp_size);
    if (d->n_kv_heads < 1 || d->n_kv_heads > d->n_heads)
      return fail(TPSLICE_ERR_SHAPE, "n_kv_heads %d outside [1, n_heads]", d->n_kv_heads);
    if (d->n_kv_heads >= d->tp_size && d->n_kv_heads % d->tp_size)
      return fail(TPSLICE_ERR_SHAPE, "%d kv heads do not split over tp_size %d", d->n_kv_heads, d->tp_size);
    qh = d->n_heads / d->tp_size;
    kvh = d->n_kv_heads >= d->tp_size ? d->n_kv_heads / d->tp_size : 1;
  }
  const int64_t M = d->tokens, h = d->hidden;
  const int64_t N1 = d->act == TPSLICE_ACT_SWIGLU ? 2 * Fp : Fp;
  const int64_t qkv = int64_t(qh + 2 * kvh) * d->head_dim, ctx = int64_t(qh) * d->head_dim;
  if (!fits_4g(M, h, 2) || !fits_4g(M, N1, 2) || !fits_4g(N1, h, 2) || !fits_4g(h, Fp, 2) ||
      !fits_4g(M, qkv, 2) || !fits_4g(qkv, h, 2) || !fits_4g(M, ctx, 2) || !fits_4g(h, ctx, 2))
    return fail(TPSLICE_ERR_SHAPE, "an operand exceeds 4 GiB");

  tpslice_plan_s* p = new (std::nothrow) tpslice_plan_s();
  if (!p) return fail(TPSLICE_ERR_INVALID, "out of host memory");
  p->magic = kPlanMagic;
  p->desc = *d;
  p->M = M; p->h = h; p->Fp = Fp; p->N1 = N1; p->qkv = qkv; p->ctx = ctx;
  p->r = d->n_row_slices; p->c = d->n_col_slices;
  if (p->r == 0 || p->c == 0) choose_slices(d, Fp, N1, qkv, ctx, &p->r, &p->c);
  p->desc.n_row_slices = p->r;
  p->desc.n_col_slices = p->c;
  p->Ms = M / p->r; p->hc = h / p->c;
  p->pc = (p->c > 1 && (d->flags & TPSLICE_F_HANDOFF_ROWS)) ? 1 : p->c;
  p->pw = h / p->pc;
  // The up-projection and dH are not handed off (the down-projection and dX after them are): each
  // runs over groups of row slices, the fewest whose product comes within 5% of the best time per
  // row slice, with the whole batch's k split, so that every slicing of the same batch sums k in
  // the same order. On the 70B shard a 2048-row slice's dH is 112 tiles of 256 x 256 (44% of the
  // CUs); two row slices make 224, with no split and no reduction pass. On the 13B shard a row
  // slice's up-projection is 128 tiles of 256 x 224; all four make 512.
  p->qh = qh; p->kvh = kvh;
  forward_schedule(p);
  p->sp_dh = choose_split(M, Fp, h);
  p->gdh = slice_group(p->r, p->Ms, Fp, h, kDgrad, d->act == TPSLICE_ACT_SWIGLU ? kEpiDswiglu : kEpiDgelu,
                       p->sp_dh);
  for (const int32_t want : {d->up_group, d->dh_group}) {
    if (want > 0 && p->r % want != 0) {
      const int32_t r = p->r;
      delete p;
      return fail(TPSLICE_ERR_INVALID, "a group of %d row slices does not divide the %d row slices", want, r);
    }
  }
  if (d->dh_group > 0) p->gdh = d->dh_group;
  const bool serial = d->flags & TPSLICE_F_SERIALIZE;
  p->E = serial ? 1 : (d->n_copy_streams ? d->n_copy_streams : 1);
  // One worker stream: it is the caller's stream. A worker stream of its own would only add a
  // fork and a join per call (about 13 us at each call boundary; GPT-3 2.7B MLP chain 1095 ->
  // 1123 TFLOP/s on the same GPU), since the caller waits for the products anyway.
  if (p->S == 1 && !serial) p->desc.flags |= TPSLICE_F_CALLER_WORKER;
  p->qh = qh; p->kvh = kvh;
  p->trace = 0;
  p->rt = nullptr;
  // k splits of the products over all tokens (each a function of that product's shape only); the
  // weight gradients may split only their last rows
  const SplitChoice s_dw1 = choose_split_tail(N1, h, M), s_dw2 = choose_split_tail(h, Fp, M);
  const SplitChoice s_dwo = qh ? choose_split_tail(h, ctx, M) : SplitChoice{1, 0};
  const SplitChoice s_dwqkv = qh ? choose_split_tail(qkv, h, M) : SplitChoice{1, 0};
  p->sp_dw1 = s_dw1.splits; p->tl_dw1 = s_dw1.tail_rows;
  p->sp_dw2 = s_dw2.splits; p->tl_dw2 = s_dw2.tail_rows;
  p->sp_dc = qh ? choose_split(M, ctx, h) : 1;
  p->sp_dwo = s_dwo.splits; p->tl_dwo = s_dwo.tail_rows;
  p->sp_dwqkv = s_dwqkv.splits; p->tl_dwqkv = s_dwqkv.tail_rows;
  // QKV over all tokens runs alone (after the slices), where the forward-only tiles that fill the
  // last round compete with a split of 256 x 256 tiles: the split only when the model prefers it
  if (qh) {
    const int s = choose_split(M, qkv, h);
    p->sp_qkv = s > 1 && estimate_product_us(M, qkv, h, kFwd, kEpiBf16, true, s) <
                             estimate_product_us(M, qkv, h, kFwd, kEpiBf16, true, 1) ? s : 1;
  } else {
    p->sp_qkv = 1;
  }
  // Products of adjacent row slices share the GPU on two worker streams. A compute unit holding a
  // 128 x 128 block (64 KB of LDS) has no room for a four-wave 256 x 256 block (128 KB) of the
  // product beside it, so mixing the two leaves units waiting: when the row slices' first product
  // takes the four-wave tile, every product is asked for it (those it cannot take fall back to
  // their own choice). Measured with 2048-row slices: Llama-2 7B MLP 937 TFLOP/s against 891 with
  // 128 x 128 down-projection pieces beside four-wave up-projections; Llama-3 70B layer 1062
  // against 984.
  p->tile = int32_t((d->flags & TPSLICE_F_TILE_MASK) >> TPSLICE_F_TILE_SHIFT);
  if (p->tile == kTileAuto && p->S > 1 &&
      choose_tile(p->Ms, Fp, h, kFwd, d->act == TPSLICE_ACT_SWIGLU ? kEpiSwiglu : kEpiGelu, false) ==
          kTile256x256w4)
    p->tile = kTile256x256w4;
  *out = p;
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_plan_info(tpslice_plan_t p, tpslice_plan_info_t* info) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (!info) return fail(TPSLICE_ERR_INVALID, "info is NULL");
  info->tokens = p->M; info->hidden = p->h; info->ffn_shard = p->Fp; info->n1 = p->N1;
  info->qkv_width = p->qkv; info->ctx_width = p->ctx;
  info->rows_per_slice = p->Ms; info->handoff_cols = p->hc;
  info->n_row_slices = p->r; info->n_col_slices = p->c;
  info->n_streams = p->S; info->n_copy_streams = p->E;
  info->q_heads = p->qh; info->kv_heads = p->kvh;
  const int32_t sp[8] = {p->sp_up, p->sp_qkv, p->sp_dh, p->sp_dw1, p->sp_dw2, p->sp_dc, p->sp_dwo, p->sp_dwqkv};
  for (int k = 0; k < 8; ++k) info->k_splits[k] = sp[k];
  // rows each split covers: a tail split's last rows, else the product's rows
  const int64_t rows[8] = {int64_t(p->Ms) * p->gup, p->M, int64_t(p->Ms) * p->gdh,
                           p->tl_dw1 ? p->tl_dw1 : p->N1, p->tl_dw2 ? p->tl_dw2 : p->h, p->M,
                           p->tl_dwo ? p->tl_dwo : p->h, p->tl_dwqkv ? p->tl_dwqkv : p->qkv};
  for (int k = 0; k < 8; ++k) info->k_split_rows[k] = sp[k] > 1 ? int32_t(rows[k]) : 0;
  const double gbps = p->desc.handoff_gbps > 0.0f ? double(p->desc.handoff_gbps) : kLocalHandoffGbps;
  info->dh_group_slices = p->gdh;
  info->up_group_slices = p->gup;
  info->predicted_forward_us =
      predict_forward_us(&p->desc, p->Fp, p->N1, p->qh ? p->qkv : 0, p->ctx, p->r, p->c, p->S, p->gup, gbps);
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_plan_piece(tpslice_plan_t p, int32_t index, int64_t out[4]) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (!out) return fail(TPSLICE_ERR_INVALID, "out is NULL");
  if (index < 0 || index >= p->r * p->c)
    return fail(TPSLICE_ERR_INVALID, "piece %d outside [0, %d)", index, p->r * p->c);
  const int32_t i = index / p->c, j = index % p->c;
  out[0] = int64_t(i) * p->Ms;
  out[1] = int64_t(i + 1) * p->Ms;
  out[2] = int64_t(j) * p->hc;
  out[3] = int64_t(j + 1) * p->hc;
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_workspace_size(tpslice_plan_t p, int32_t op, size_t* bytes) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (!bytes) return fail(TPSLICE_ERR_INVALID, "bytes is NULL");
  switch (op) {
    case TPSLICE_OP_MLP_FWD: *bytes = mlp_fwd_ws(p).total; return TPSLICE_OK;
    case TPSLICE_OP_MLP_BWD: *bytes = mlp_bwd_ws(p).total; return TPSLICE_OK;
    case TPSLICE_OP_ATTNPROJ_FWD: *bytes = attn_fwd_ws(p).total; return TPSLICE_OK;
    case TPSLICE_OP_ATTNPROJ_BWD: *bytes = attn_bwd_ws(p).total; return TPSLICE_OK;
    case TPSLICE_OP_ATTN_CORE_BWD: *bytes = p->qh ? attn_bwd_workspace_bytes(p->M, p->qh, p->kvh) : 0; return TPSLICE_OK;
    default: return fail(TPSLICE_ERR_INVALID, "unknown op %d", op);
  }
}

extern "C" const char* tpslice_error_string(tpslice_status_t s) {
  switch (s) {
    case TPSLICE_OK: return "ok";
    case TPSLICE_ERR_INVALID: return "invalid argument";
    case TPSLICE_ERR_SHAPE: return "unsupported shape";
    case TPSLICE_ERR_UNSUPPORTED: return "unsupported request";
    case TPSLICE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case TPSLICE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char* tpslice_last_error(void) { return tps::g_last_error; }
