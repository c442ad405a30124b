// Internal launch interface of the bf16 MFMA GEMM family (gfx950).
//
// C[m][n] = sum_k A(m, k) * B(k, n), fp32 accumulation, fused epilogue. Operand storage:
//   kFwd   : A(m,k) = A[m*lda + k]   B(k,n) = B[n*ldb + k]   (both read along k)
//   kDgrad : A(m,k) = A[m*lda + k]   B(k,n) = B[k*ldb + n]
//   kWgrad : A(m,k) = A[k*lda + m]   B(k,n) = B[k*ldb + n]
// Requirements (checked by the caller): M, N, K >= 0; N, K multiples of 8; for kWgrad M a
// multiple of 8; every operand below 4 GiB; 16-byte aligned pointers and leading dimensions that
// are multiples of 8 elements.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tps {

enum GemmLayout : int { kFwd = 0, kDgrad = 1, kWgrad = 2 };

enum GemmEpi : int {
  kEpiBf16 = 0,    // C = bf16(acc + bias)                                     bias [N] or null
  kEpiGelu = 1,    // U = acc + bias; aux_out = bf16(U) (if set); C = bf16(gelu(U))
  kEpiSwiglu = 2,  // B rows n and half+n give G and V; aux_out[., n | half+n] = bf16(G | V)
                   // (if set); C = bf16(silu(G) * V)
  kEpiDgelu = 3,   // U = aux_in; C = bf16(acc * gelu'(U)); aux_out = bf16(gelu(U))
  kEpiDswiglu = 4, // G, V = aux_in[., n], aux_in[., half+n]; C[., n] = bf16(acc V silu'(G)),
                   // C[., half+n] = bf16(acc silu(G)); aux_out = bf16(silu(G) V)
  kEpiF32 = 5,     // C (fp32) = acc, or C + acc when accumulate (C loaded into the accumulator
                   // before the k loop, so a run split along k reproduces the unsplit sums)
  kEpiPartialDual = 6  // split-k partial of a SwiGLU product: C (fp32) [., n] = gate sums,
                       // C[., half+n] = up sums (internal to the split path)
};

struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  const void* bias;
  const void* aux_in;
  void* aux_out;
  int64_t lda, ldb, ldc, ld_in, ld_out;
  int64_t half;        // column offset of the second half (SwiGLU epilogues)
  int32_t M, N, K;     // N: output columns (SwiGLU: F')
  int32_t accumulate;  // kEpiF32 only
  // filled by launch_gemm
  uint32_t a_bytes, b_bytes;
  int32_t tiles_m, tiles_n;
  int32_t splits;         // k splits (1: none); split s covers k blocks [s kb_split, (s+1) kb_split)
  int32_t kb_split;       // 64-wide k blocks per split
  int64_t part_stride;    // floats between the fp32 partial products of consecutive splits
};

// Block tile of a launch. Every tile reduces k in the same order, so the choice never changes a
// result bit. The 320-wide tiles take only products whose operands are both read along k, without
// the SwiGLU pairing, the four-wave tiles only products with K a multiple of 64 that do not
// accumulate into an fp32 output (256 x 320: forward only; 256 x 160: forward, and activation
// gradients with a bf16 or GeLU-gradient epilogue); a request a tile cannot serve falls back to
// kTileAuto.
enum GemmTile : int {
  kTileAuto = 0,
  kTile256x256 = 1,
  kTile128x128 = 2,
  kTile256x320 = 3,
  kTile128x320 = 4,
  kTile128x256 = 5,
  kTile128x128w8 = 6,  // 128 x 128 with 8 waves, one block per CU
  kTile256x256w4 = 7,  // 256 x 256 with 4 waves and a software-pipelined loop: products with K a
                       // multiple of 64 and no accumulation into an fp32 output
  kTile256x160w4 = 8,  // 256 x 160, likewise, forward products without the SwiGLU pairing and
                       // activation gradients with a bf16 or GeLU-gradient epilogue (their B tile
                       // padded to 256 columns in LDS)
  kTile256x320w4 = 9,  // 256 x 320, likewise, forward products without the pairing (accumulators
                       // partly in VGPRs)
  kTile256x224w4 = 10, // 256 x 224 (112 gate + 112 up columns), 4 waves along m: forward SwiGLU only
  kTileCount = 11
};

// The tile kTileAuto resolves to for an M x N x K product (N: output columns). `alone`: the product
// has the GPU to itself (no products of other slices run beside it), so tiles that fill the last
// round of blocks are worth their lower per-CU rate. `fill` (optional) receives the share of the
// block slots the chosen tile occupies over its rounds.
// `accumulate`: an fp32 output is added to (the four-wave tiles do not take these).
int choose_tile(int64_t M, int64_t N, int64_t K, int layout, int epi, bool alone, double* fill = nullptr,
                bool accumulate = false);

// The kernel of the latest GEMM launch from this thread (launch_gemm, or the partial product of
// launch_gemm_split): its Tile<BM, BN, waves_m, waves_n, blocks_per_cu> parameters, layout and
// epilogue, and its grid (blocks of `threads` work-items). Traces name each launch's kernel by it.
struct LaunchInfo {
  int32_t bm = 0, bn = 0, waves_m = 0, waves_n = 0, blocks_per_cu = 0, layout = 0, epi = 0;
  int32_t blocks = 0, threads = 0;
};
LaunchInfo last_launch();

// Queue one GEMM on `stream`. With `start`/`stop` events the launch records the kernel's own start
// and end times in them (timestamps of the dispatch itself, no extra marker packets).
// Returns hipSuccess or the launch error.
hipError_t launch_gemm(GemmArgs g, int layout, int epi, hipStream_t stream, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr, int tile = kTileAuto, bool alone = false);

// Products whose k is long and whose output is small leave most CUs idle (a weight gradient over
// all tokens with a narrow output, a thin slice of a narrow projection). Split-k: the k blocks are
// cut into `splits` equal runs, each run's fp32 product goes to its own partial buffer, and a
// reduction kernel adds the partials in split order and applies the product's epilogue (bias,
// activation, saved pre-activation, activation gradient; for kEpiF32 after the existing output
// when accumulating). Every run of the same product with the same split count gets the same bits;
// the sums differ in rounding from an unsplit product.
// choose_split: split count for an M x N x K product (N: output columns; SwiGLU: both halves).
int choose_split(int64_t M, int64_t N, int64_t K);
// A split of only the last rows of a product ("tail split"): the first M - tail_rows rows (a
// multiple of 256) run unsplit in whole rounds of 256 x 256 tiles, and the tiles of the remaining
// rows, which would leave the last round partly empty, run split along k into a full round. Each
// output element still gets one fixed summation order (its rows' part decides which), so every run
// of the same product shape gets the same bits. tail_rows == 0: the split (if any) covers the whole
// product, as choose_split decides.
struct SplitChoice {
  int splits;         // 1: no split
  int64_t tail_rows;  // rows the split covers (the last ones); 0: all of them
};
// For an M x N x K weight-gradient product (both operands read across k; 256 x 256 tiles): the
// whole-product split of choose_split, or a tail split when the same cost model (rounds of 256
// CUs x k blocks per run, the reduction's HBM passes, a launch) puts it at least 5% below.
SplitChoice choose_split_tail(int64_t M, int64_t N, int64_t K);
// Split count of a per-slice product. It must not depend on the slice height, or slicing would
// change a product's rounding; it is chosen for 2048-row slices (the workloads' slice height).
constexpr int64_t kSplitRefRows = 2048;
inline int choose_slice_split(int64_t N, int64_t K) { return choose_split(kSplitRefRows, N, K); }
// Estimated time (us) of one M x N x K product on this GPU (N: output columns; SwiGLU: of each
// half; not `alone`: two products of M / 2 rows side by side), with the tile choose_tile picks and
// `splits` k splits (1: none), from the same per-tile cost model: rounds of 256 CUs times the k
// blocks per run at about 1.9 us per 64-wide k block of a 256 x 256 tile, plus the split
// reduction's HBM passes and a fixed launch cost. Used to compare slicings, not as a timing.
double estimate_product_us(int64_t M, int64_t N, int64_t K, int layout, int epi, bool alone, int splits = 1);
// Bytes of partial buffers of an M x N product (N: both halves for SwiGLU) split `splits` ways
// (0 when splits == 1).
size_t split_partials_bytes(int64_t M, int64_t N, int splits);
// Queue a split product: the GEMM into `partials` (fp32), then the reduction with epilogue `epi`
// into g's outputs, on `stream`. When tracing, `start`/`gemm_stop` bracket the GEMM and
// `gemm_stop`/`stop` the reduction. The partial products
// run 256 x 256 tiles: the four-wave pipelined ones when K is a multiple of 64 and `tile` is
// kTileAuto or kTile256x256w4, else the eight-wave ones (the same bits).
// tail_rows in (0, M) with M - tail_rows a multiple of 256: a tail split (choose_split_tail). The
// partial products of the last tail_rows rows run first, then the unsplit product of the other
// rows (launch_gemm with `tile`), then the reduction of the tail rows; `partials` holds the tail's
// partials only, and `gemm_stop` marks the end of the unsplit part. Not for SwiGLU products.
hipError_t launch_gemm_split(GemmArgs g, int layout, int epi, int splits, float* partials, hipStream_t stream,
                             hipEvent_t start = nullptr, hipEvent_t stop = nullptr, int tile = kTileAuto,
                             hipEvent_t gemm_stop = nullptr, int64_t tail_rows = 0);

// A one-wave kernel that does nothing. Queued on a stream after DMA-engine copies it completes only
// after them (stream order), so an event recorded after it marks the copies' completion.
hipError_t launch_fence(hipStream_t stream);

constexpr int kColsumChunkRows = 256;

// Column sums of a bf16 [M][N] matrix into fp32 out[N] (out += sums when accumulate), in a fixed
// order: partial sums over 256-row chunks into `partials` ([ceil(M/256)][N] fp32), then the chunks
// in ascending order.
hipError_t launch_colsum(const void* X, int64_t ldx, int32_t M, int32_t N, float* partials, float* out,
                         int32_t accumulate, hipStream_t stream);
size_t colsum_partials_bytes(int32_t M, int32_t N);

}  // namespace tps
