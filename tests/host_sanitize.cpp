// Host-side checks of the library under AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU
// work: plans over a grid of descriptors (valid and invalid), their info, workspace sizes and
// pieces, argument errors of every entry point, the two-strand schedule on random profiles, and the
// error strings. Built host-only (no device code) against the library's sources by
// tests/test_host_sanitizers.py; prints "ok" and exits 0 when every check passes.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "tpslice.h"

static int g_fail = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                           \
    }                                                                     \
  } while (0)

static void exercise_plan(tpslice_plan_t p) {
  tpslice_plan_info_t info;
  CHECK(tpslice_plan_info(p, &info) == TPSLICE_OK);
  CHECK(tpslice_plan_info(p, nullptr) == TPSLICE_ERR_INVALID);
  const int32_t n = info.n_row_slices * info.n_col_slices;
  int64_t prev_end = -1;
  for (int32_t i = -1; i <= n; ++i) {
    int64_t out[4] = {0, 0, 0, 0};
    const tpslice_status_t st = tpslice_plan_piece(p, i, out);
    if (i < 0 || i >= n) {
      CHECK(st != TPSLICE_OK);
      continue;
    }
    CHECK(st == TPSLICE_OK);
    CHECK(out[0] >= 0 && out[0] <= out[1] && out[1] <= info.tokens);
    CHECK(out[2] >= 0 && out[2] < out[3] && out[3] <= info.hidden);
    (void)prev_end;
  }
  for (int32_t op = -1; op <= 5; ++op) {
    size_t bytes = 0;
    const tpslice_status_t st = tpslice_workspace_size(p, op, &bytes);
    CHECK(op < 0 || op > 4 ? st != TPSLICE_OK : st == TPSLICE_OK);
  }
  // argument errors, detected before any GPU work
  CHECK(tpslice_mlp_fwd(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) !=
        TPSLICE_OK);
  CHECK(tpslice_mlp_bwd(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        2, nullptr, 0, nullptr) != TPSLICE_OK);
  CHECK(tpslice_attnproj_fwd(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                             nullptr) != TPSLICE_OK);
  CHECK(tpslice_attnproj_bwd(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr) != TPSLICE_OK);
  CHECK(tpslice_attn_core_fwd(p, nullptr, nullptr, nullptr, 0, nullptr) != TPSLICE_OK);
  CHECK(tpslice_attn_core_bwd(p, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr) != TPSLICE_OK);
  CHECK(tpslice_mlp_fwd_static(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) !=
        TPSLICE_OK);
  if (info.tokens > 0) CHECK(tpslice_handoff_copy(p, nullptr, nullptr, nullptr) != TPSLICE_OK);
  int32_t count = -1;
  CHECK(tpslice_trace_read(p, nullptr, 0, &count) == TPSLICE_ERR_INVALID);  // tracing is off
  CHECK(std::strlen(tpslice_last_error()) > 0);
}

int main() {
  int plans = 0, refused = 0;
  const int64_t tokens[] = {0, 8, 64, 256, 2048, 16384};
  const int64_t hidden[] = {8, 64, 520, 8192};
  const int64_t ffn[] = {8, 264, 28672};
  const int32_t tp[] = {1, 2, 8};
  const int32_t rs[] = {0, 1, 2, 8, 16};
  const int32_t cs[] = {0, 1, 2, 4};
  const int32_t heads[][3] = {{0, 0, 0}, {8, 2, 64}, {64, 8, 128}};
  const uint32_t flags[] = {0u, TPSLICE_F_PIPELINE, TPSLICE_F_SERIALIZE, TPSLICE_F_HANDOFF_ROWS | TPSLICE_F_PIPELINE,
                            TPSLICE_F_CALLER_WORKER, TPSLICE_F_TILE(7), TPSLICE_F_TILE(11), 0x80u};
  const int32_t groups[] = {0, 1, 2, 3};
  std::mt19937 rng(7);
  for (int64_t M : tokens)
    for (int64_t h : hidden)
      for (int64_t F : ffn)
        for (int32_t t : tp)
          for (int32_t r : rs)
            for (int32_t c : cs) {
              // a random sample of the remaining dimensions per geometry keeps the run short
              tpslice_desc_t d;
              std::memset(&d, 0, sizeof(d));
              d.tokens = M; d.hidden = h; d.ffn = F; d.tp_size = t;
              d.n_row_slices = r; d.n_col_slices = c;
              const auto& hd = heads[rng() % 3];
              d.n_heads = hd[0]; d.n_kv_heads = hd[1]; d.head_dim = hd[2];
              d.act = int32_t(rng() % 3);  // includes an invalid activation id
              d.n_streams = int32_t(rng() % 4);
              d.n_copy_streams = int32_t(rng() % 3);
              d.flags = flags[rng() % 8];
              d.handoff_gbps = (rng() % 2) ? 25.0f : 0.0f;
              d.dh_group = groups[rng() % 4];
              d.up_group = groups[rng() % 4];
              tpslice_plan_t p = nullptr;
              const tpslice_status_t st = tpslice_plan(&d, &p);
              if (st != TPSLICE_OK) {
                CHECK(p == nullptr);
                CHECK(std::strlen(tpslice_last_error()) > 0);
                ++refused;
                continue;
              }
              ++plans;
              exercise_plan(p);
              CHECK(tpslice_plan_destroy(p) == TPSLICE_OK);
            }
  CHECK(tpslice_plan(nullptr, nullptr) == TPSLICE_ERR_INVALID);
  CHECK(tpslice_plan_destroy(nullptr) == TPSLICE_OK);
  CHECK(plans > 100 && refused > 100);
  // the two-strand schedule on random profiles, up to 40 x 40 segments
  for (int trial = 0; trial < 200; ++trial) {
    const int nf = int(rng() % 41), nb = int(rng() % 41);
    std::vector<double> P(size_t(nf + 1) * size_t(nb + 1));
    std::uniform_real_distribution<double> u(0.1, 3.0);
    for (double& v : P) v = u(rng);
    P[0] = 0.0;
    std::vector<int32_t> steps(size_t(2) * size_t(nf + nb + 1));
    int32_t n = -1;
    double t = -1.0;
    CHECK(tpslice_strand_schedule(P.data(), nf, nb, steps.data(), &n, &t) == TPSLICE_OK);
    CHECK(n >= (nf > nb ? nf : nb) && n <= nf + nb && t >= 0.0);
  }
  double bad[4] = {0.0, -1.0, 1.0, 1.0};
  int32_t steps[8], n;
  double t;
  CHECK(tpslice_strand_schedule(bad, 1, 1, steps, &n, &t) == TPSLICE_ERR_INVALID);
  CHECK(tpslice_strand_schedule(bad, -3, 1, steps, &n, &t) == TPSLICE_ERR_SHAPE);
  // every status code, and the codes the enumeration's range leaves unused
  for (int code = 0; code < 8; ++code) CHECK(tpslice_error_string(tpslice_status_t(code)) != nullptr);
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("ok: %d plans, %d descriptors refused\n", plans, refused);
  return 0;
}
