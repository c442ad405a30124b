// bf16 MFMA GEMM family for gfx950 (MI355X) with fused layer epilogues.
//
// One kernel template serves a family of block tiles (k step 64, v_mfma_f32_16x16x32_bf16, fp32
// accumulators, two waves per SIMD so one wave's waits hide under the other's MFMAs):
//   * 256 x 256, 8 waves (2 x 4), each wave 128 x 64 outputs, one block per CU (128 KB LDS);
//   * 256 x 320 and 128 x 320, 8 waves, waves of 128 x 80 / 64 x 80 (products whose operands are
//     both read along k, without the SwiGLU pairing), one block per CU;
//   * 128 x 256, 8 waves, waves of 64 x 64, one block per CU (96 KB LDS);
//   * 128 x 128, 4 waves (2 x 2), waves of 64 x 64, two blocks per CU (64 KB LDS each);
//   * 256 x 256, 256 x 160 and 256 x 320 with 4 waves (2 x 2, one wave per SIMD), waves of
//     128 x 128 / 128 x 80 / 128 x 160, and 256 x 224 with 4 waves stacked along m (64 x 224,
//     forward SwiGLU only), one block per CU, for products with k a multiple of 64 (256 x 256 in
//     every operand layout and for split runs; 256 x 320 forward only; 256 x 160 forward and the
//     activation gradients with a bf16 or GeLU-gradient epilogue, whose B tile, read across k, is
//     padded to 256 columns in LDS): a software-pipelined loop (barrier between the two k steps,
//     loads two blocks ahead, LDS reads and load issue interleaved one by one with the MFMAs) that
//     leaves no wait to another wave.
// The launcher picks per product the tile with the smallest estimated time on 256 CUs: whole
// rounds of resident blocks times the tile's work over its measured per-CU rate. Larger tiles move
// fewer bytes per flop; the others cut the last, partly filled round (e.g. a 4096 x 5120 product is
// 320 tiles of 256 x 256 - two rounds, the second a quarter full - but exactly 256 tiles of
// 256 x 320). Every tile reduces k in the same order (ascending 64-wide blocks, two 32-wide MFMA
// steps each), so every output element gets bitwise the same sum whichever tile, slicing or tile
// position produced it.
// Operand tiles go global -> LDS by direct loads (buffer_load_dwordx4 ... lds) into two LDS stages:
// block k+1 loads while block k is multiplied, and the load instructions are spread between the
// first MFMAs of the block instead of being issued together after the barrier. 16-byte XOR
// swizzles keep LDS traffic at full rate (chosen by measuring each candidate pattern's LDS
// throughput on gfx950):
//   * an operand read along k ("KC") is kept as [rows][64 k] (128-byte rows), fragments read
//     with ds_read_b128;
//   * an operand read across k ("NC", rows of k in memory) is kept as [64 k][tile columns] and
//     its fragments come from ds_read_b64_tr_b16, which transposes 16-bit elements across each
//     16-lane group: result element v of lane i is element i%4 of the 8 bytes addressed by
//     group lane 4v + (i%16)/4.
// The MFMA is issued with the B fragment first, so each lane ends up holding four consecutive
// output columns of one row: lane l, register v of tile (im, in) is
//   C[row0 + 16 im + l%16][col0 + 16 in + 4 (l/16) + v].
// Loads go through buffer resources: for tiles wholly inside the operands the k offset rides in
// the scalar offset (no per-lane work); edge tiles and the last partial k block use per-chunk
// offsets and the range check, which returns zeros outside the operand.
// Tiles are numbered so that each XCD (workgroups are dispatched round-robin over the 8 XCDs)
// receives a contiguous run of the grouped tile order, which keeps the operand rows and columns a
// run shares in that XCD's L2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "gemm.hpp"

namespace tps {

constexpr int kBKTile = 64;
// Block tile: BM x BN (BN counts B-tile columns; SwiGLU products hold gate and up halves),
// waves in a WM x WN grid, `blocks` resident blocks per CU.
template <int BM_, int BN_, int WM, int WN, int BLOCKS>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, kWavesM = WM, kWavesN = WN, kBlocksPerCU = BLOCKS;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int kWaveM = BM / WM;             // output rows per wave
  static constexpr int kFM = kWaveM / 16;            // MFMA tiles per wave along m
  static constexpr int kFN = BN / WN / 16;           // MFMA tiles per wave along n
  static constexpr int kATileBytes = BM * kBKTile * 2, kBTileBytes = BN * kBKTile * 2;
  static constexpr int kStageBytes = kATileBytes + kBTileBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;  // two operand stages
  static constexpr int kARuns = kATileBytes / 1024 / kWaves;  // 1-KB load runs per wave
  static constexpr int kBRuns = kBTileBytes / 1024 / kWaves;
  // an operand read across k is staged as [64 k][tile columns]: a 1-KB load run must hold whole
  // k rows, and the SwiGLU pairing needs an even number of MFMA columns per wave
  static constexpr bool kNcA = 1024 % (BM * 2) == 0;
  static constexpr bool kDualOk = kFN % 2 == 0;
  // LDS columns of a B tile read across k: BN itself when its k rows fill 1-KB runs whole, else
  // (four-wave tiles narrower than 256, e.g. 256 x 160 on activation gradients) 256, the columns
  // past BN loaded but never read, so that the runs and the conflict-free swizzle of 256-column
  // rows serve it unchanged; 0: none
  static constexpr int kBnL = 1024 % (BN * 2) == 0 ? BN : (WM * WN == 4 && BM == 256 && BN < 256) ? 256 : 0;
  static constexpr bool kNcB = kBnL > 0;
  static constexpr int kBNcTileBytes = kBnL * kBKTile * 2;
  static_assert(kARuns >= 1 && kBRuns >= 1 && kATileBytes % (1024 * kWaves) == 0 &&
                kBTileBytes % (1024 * kWaves) == 0, "tiles load in whole 1-KB runs per wave");
  static_assert(kLdsBytes * BLOCKS <= 160 * 1024 && 2 * (kATileBytes + kBNcTileBytes) * BLOCKS <= 160 * 1024,
                "LDS per CU");
};
// Operand stage and LDS bytes of a tile in one operand layout (a B tile read across k may be wider
// in LDS than in the product)
template <class TL, int LAYOUT>
constexpr int stage_bytes() { return TL::kATileBytes + (LAYOUT == kFwd ? TL::kBTileBytes : TL::kBNcTileBytes); }
template <class TL, int LAYOUT>
constexpr int lds_bytes() { return 2 * stage_bytes<TL, LAYOUT>(); }
using TileL = Tile<256, 256, 2, 4, 1>;
using TileS = Tile<128, 128, 2, 2, 2>;
using TileW = Tile<256, 320, 2, 4, 1>;
using TileN = Tile<128, 320, 2, 4, 1>;
using TileM = Tile<128, 256, 2, 4, 1>;
using TileT = Tile<128, 128, 2, 4, 1>;
// Four waves, one per SIMD, each 128 rows x (BN / 2) columns, with the software-pipelined main
// loop (gemm_kernel); for products whose K is a multiple of 64. 256 x 160 serves forward products
// and activation gradients with a bf16 or GeLU-gradient epilogue (its B tile, read across k there,
// padded to 256 columns in LDS): a 2048-row slice of a 5120-wide output makes 8 x 32 = 256 blocks,
// one per CU, where 256 x 256 makes 160.
using TileL4 = Tile<256, 256, 2, 2, 1>;
using TileH4 = Tile<256, 160, 2, 2, 1>;
// 256 x 320 with four waves of 128 x 160: 320 accumulator registers per lane, more than the 256
// AGPRs, so the last accumulator columns live in VGPRs (the MFMA takes either)
using TileW4 = Tile<256, 320, 2, 2, 1>;
// 256 x 224 with four waves stacked along m (64 x 224 each), forward SwiGLU products only: 112 gate
// and 112 up columns per block, so a 2048-row slice of a 3584-wide FFN shard makes 8 x 32 = 256
// blocks, one per CU, where 256 x 256 makes 224 (the Llama-3 70B shard's up-projection)
using TileG4 = Tile<256, 224, 4, 1, 1>;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;                          // k per block
constexpr int kRowBytes = kBK * 2;               // KC tile row: 128 bytes
constexpr int kChunks = kBK / 8;                 // 16-byte chunks per KC row
constexpr int kRowsPerRun = 1024 / kRowBytes;    // KC rows per 1-KB load run
constexpr int kGroupM = 4;                       // tile rows per group of the tile order
constexpr int kCUs = 256;
// Cache policy of the operand loads: the sc1 scope bit. The tiles stream through each CU once
// (the vector L1 cannot hold them between uses), and with this bit the direct-to-LDS loads run
// 3-7% faster on gfx950 than with the default policy (measured on 8192^3 and Llama-shaped products).
constexpr int kLoadPolicy = 16;
constexpr uint32_t kOob = 0xFFFFF000u;           // buffer offset that reads as zero: operands are
                                                 // smaller than 4 GiB - 4 KiB


typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The same descriptor as raw words, for the pipelined loop's own load instruction (dword1: the
// high address bits, stride 0; dword3: the flags make_rsrc passes).
__device__ inline i32x4 raw_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xffffu), int(bytes), 0x00020000};
}

// One direct global -> LDS load (buffer_load_dwordx4 ... lds, sc1): lane l's 16 bytes at
// voff + soff go to LDS byte address lds + 16 l. It is written out here rather than through the
// builtin because the compiler, which cannot tell which LDS bytes such a load writes, makes every
// later ds_read_b64_tr_b16 wait for all loads in flight (s_waitcnt vmcnt(0)); in the pipelined loop
// that serializes the next block's loads behind each transposing read. The loop's own waits
// (s_waitcnt vmcnt(0) before the barrier that publishes a stage) order these loads against the
// reads. M0 carries the LDS address and is restored afterwards; the load writes no register.
// f(integral_constant<int, i>) for i = I .. N-1, in order
template <int I, int N, class F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// `lds` (wave-uniform) + OFF is the LDS address.
template <int OFF>
__device__ inline void dma16(const i32x4& rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %5\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen sc1 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff), "i"(OFF)
      : "memory", "scc");
}

// 16-byte chunk swizzles, chosen by measurement on gfx950 (LDS read throughput of each candidate
// lane pattern): KC rows of 128 B (8 chunks) XOR the chunk with ((r >> 1) & 7) ^ ((r & 1) << 2),
// which lets the fragment reads (16 consecutive rows per 16-lane group) run at full LDS rate;
// NC rows XOR with (k & 3) << 1 | (k >> 3 & 1) << 3 for the transpose reads (each 32-lane half of
// a read touches 8 k rows x 32 bytes, which this spreads over all 64 banks for 256- and 512-byte
// rows alike).
__device__ inline int swz_kc(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ inline int swz_nc(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

__device__ inline float bf2f(unsigned short b) { return __uint_as_float(uint32_t(b) << 16); }

// Activation math, in few VALU instructions: the epilogue's fp32 vector work runs after the MFMA
// loop and is paid per output element, so the library erff (two polynomial branches) and the
// correctly rounded division cost a fifth of a GeLU product's time.
//
// Normal upper tail Q(a) = P(Z > a) = erfc(a / sqrt 2) / 2 for a = |u|, by the rational
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2), t = 1 / (1 + p x), absolute error
// below 1.5e-7. Here x = a / sqrt 2, so p becomes p / sqrt 2 and exp(-x^2) = 2^(-a^2 log2(e) / 2);
// the coefficients carry the factor 1/2. Returns Q(a) and e = exp(-u^2 / 2).
struct NormalTail { float q, e; };
__device__ inline NormalTail normal_tail(float u) {
  const float a = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(a, 0.2316418883f, 1.0f));
  float p = fmaf(t, 0.5307027145f, -0.7265760135f);
  p = fmaf(t, p, 0.7107068705f);
  p = fmaf(t, p, -0.1422483680f);
  p = fmaf(t, p, 0.1274147960f);
  const float e = __builtin_amdgcn_exp2f(u * u * -0.72134752044448170f);
  return {t * p * e, e};
}
// GeLU(u) = u Phi(u), with Phi(u) = 1 - Q(u) for u >= 0 and Q(-u) for u < 0:
// GeLU(u) = (u + |u| (1 - 2 Q(|u|))) / 2. Absolute error below 3e-7 for finite u.
__device__ inline float gelu_f(float u) {
  const NormalTail n = normal_tail(u);
  return 0.5f * fmaf(fabsf(u), fmaf(-2.0f, n.q, 1.0f), u);
}
// GeLU'(u) = Phi(u) + u phi(u), phi(u) = exp(-u^2 / 2) / sqrt(2 pi); gelu_and_grad gives both.
__device__ inline void gelu_and_grad(float u, float& h, float& d) {
  const NormalTail n = normal_tail(u);
  h = 0.5f * fmaf(fabsf(u), fmaf(-2.0f, n.q, 1.0f), u);
  d = (u >= 0.0f ? 1.0f - n.q : n.q) + u * n.e * 0.39894228040143270f;
}
// logistic sigmoid 1 / (1 + e^-g), with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ inline float sigmoid_f(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896339f));
}

__device__ inline i32x2 pack_bf16x4(float a, float b, float c, float d) {
  bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  return __builtin_bit_cast(i32x2, v);
}

__device__ inline void load_bf16x4(const void* base, int64_t elem, float (&o)[4]) {
  const i32x2 v = *reinterpret_cast<const i32x2*>(reinterpret_cast<const unsigned short*>(base) + elem);
  o[0] = __uint_as_float(uint32_t(v[0]) << 16);
  o[1] = __uint_as_float(uint32_t(v[0]) & 0xffff0000u);
  o[2] = __uint_as_float(uint32_t(v[1]) << 16);
  o[3] = __uint_as_float(uint32_t(v[1]) & 0xffff0000u);
}

__device__ inline void store_bf16x4(void* base, int64_t elem, float a, float b, float c, float d) {
  *reinterpret_cast<i32x2*>(reinterpret_cast<unsigned short*>(base) + elem) = pack_bf16x4(a, b, c, d);
}

// ------------------------------------------------------------------------------ operand staging
// Each operand tile is filled by direct global -> LDS loads (buffer_load_dwordx4 ... lds): one load
// instruction writes 64 consecutive 16-byte LDS slots (a 1-KB run), lane l into slot l. Each wave
// owns RUNS consecutive runs of each tile; each lane loads the global chunk that belongs in its
// slot, so the swizzled layout comes from the choice of global address.
//   KC tile [rows][64 k]: run s holds rows 8s..8s+7; lane l -> row 8s + l/8, slot chunk l%8.
//   NC tile [64 k][COLS]: run s holds 1024 / (2 COLS) k rows; lane l -> k row
//                         s * (1024 / (2 COLS)) + l / (COLS / 8), slot chunk l % (COLS / 8).
//                         In a padded tile (width `used` < COLS, used >= COLS / 2) the slots of
//                         columns past `used` repeat chunk ch % (COLS / 16) of the same k row, a
//                         column the same load instruction already reads; they are never read.

template <int RUNS>
struct KcLoader {
  uint32_t off[RUNS];   // byte offset of the lane's chunk at k0 = 0
  uint32_t kel[RUNS];   // k index (element) of the lane's chunk at k0 = 0
  uint32_t valid;       // bit j: the chunk's row lies inside the operand
  // dual: the tile's first half_rows rows come from row0.., the rest from half + row0..
  __device__ void init(int wave, int lane, int64_t ld, int row0, int row_limit, bool dual, int64_t half,
                       int half_rows) {
    valid = 0;
    for (int j = 0; j < RUNS; ++j) {
      const int r = (wave * RUNS + j) * kRowsPerRun + lane / kChunks;  // tile row
      const int ch = (lane % kChunks) ^ swz_kc(r);                      // logical chunk (k / 8)
      int li = r, gro;
      if (dual) {
        li = r % half_rows;
        gro = (r < half_rows) ? row0 + li : int(half) + row0 + li;
      } else {
        gro = row0 + r;
      }
      const bool ok = row0 + li < row_limit;
      off[j] = ok ? uint32_t(int64_t(gro) * ld * 2 + ch * 16) : 0u;
      kel[j] = uint32_t(ch * 8);
      valid |= uint32_t(ok) << j;
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0, int K, int j0, int j1) const {
    for (int j = j0; j < j1; ++j) {
      const bool ok = ((valid >> j) & 1) && int(kel[j]) + k0 < K;
      const uint32_t o = ok ? off[j] + uint32_t(k0) * 2 : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * RUNS + j) * 1024), 16, o, 0, 0, kLoadPolicy);
    }
  }
  // every chunk in range: k advances through the scalar offset, no per-lane arithmetic
  __device__ void issue_fast(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0, int j0, int j1) const {
    for (int j = j0; j < j1; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * RUNS + j) * 1024), 16, off[j],
                                               uint32_t(k0) * 2, 0, kLoadPolicy);
  }
};

template <int RUNS, int COLS>
struct NcLoader {
  static constexpr int kCpr = COLS / 8;               // chunks per k row
  static constexpr int kKpr = 1024 / (COLS * 2);      // k rows per run
  uint32_t col_off[RUNS];  // byte offset of the lane's chunk within a k row
  uint32_t krow[RUNS];     // tile k row of the lane's chunk
  uint32_t valid;          // bit j: the chunk's columns lie inside the operand and the tile
  uint32_t ld_bytes;
  // tile columns [col0, col0 + used), COLS / 2 <= used <= COLS
  __device__ void init(int wave, int lane, int64_t ld, int col0, int col_limit, int used) {
    valid = 0;
    ld_bytes = uint32_t(ld * 2);
    for (int j = 0; j < RUNS; ++j) {
      const int k = (wave * RUNS + j) * kKpr + lane / kCpr;
      int ch = (lane % kCpr) ^ swz_nc(k);
      if (ch * 8 >= used) ch %= kCpr / 2;
      const int c = col0 + ch * 8;
      const bool ok = c < col_limit;
      col_off[j] = ok ? uint32_t(c) * 2 : 0u;
      krow[j] = uint32_t(k);
      valid |= uint32_t(ok) << j;
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0, int K, int j0, int j1) const {
    for (int j = j0; j < j1; ++j) {
      const int k = k0 + int(krow[j]);
      const bool ok = ((valid >> j) & 1) && k < K;
      const uint32_t o = ok ? uint32_t(k) * ld_bytes + col_off[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * RUNS + j) * 1024), 16, o, 0, 0, kLoadPolicy);
    }
  }
  __device__ void issue_fast(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0, int j0, int j1) const {
    for (int j = j0; j < j1; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * RUNS + j) * 1024), 16,
                                               krow[j] * ld_bytes + col_off[j], uint32_t(k0) * ld_bytes, 0, kLoadPolicy);
  }
};

// Wait until all of this wave's buffer loads have landed, then meet the other waves. Pinned in
// place (scheduling barriers) so that MFMA work is not moved across it.
__device__ inline void wait_loads_and_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The same, also waiting for this wave's LDS reads: the pipelined loop overwrites a stage right
// after the barrier, while reads of it may still be in flight otherwise.
__device__ inline void wait_all_and_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------------------ fragment reads
// KC fragment: lane l gets operand[rb + l%16][32 kk + 8 (l/16) + 0..7].
__device__ inline bf16x8 frag_kc(const char* tile, int rb, int lane, int kk) {
  const int row = rb + (lane & 15);
  const int ch = kk * 4 + (lane >> 4);
  return *reinterpret_cast<const bf16x8*>(tile + row * kRowBytes + ((ch ^ swz_kc(row)) << 4));
}

// NC fragment: same element assignment as frag_kc, from a [64 k][COLS] tile, cb = first column.
template <int COLS>
__device__ inline bf16x8 frag_nc(const char* tile, int cb, int lane, int kk) {
  constexpr int kRow = COLS * 2;
  const int g = lane >> 4, v = (lane & 15) >> 2, q = lane & 3;
  const int chunk = (cb >> 3) + (q >> 1);
  const int k0 = kk * 32 + 8 * g + v;
  const int k1 = k0 + 4;
  const int byte_in = (q & 1) << 3;
  const char* p0 = tile + k0 * kRow + ((chunk ^ swz_nc(k0)) << 4) + byte_in;
  const char* p1 = tile + k1 * kRow + ((chunk ^ swz_nc(k1)) << 4) + byte_in;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

// ----------------------------------------------------------------------------------- epilogue
// Where the epilogue reads and writes. GlobalIO addresses row m of each operand through plain
// pointers (the split-k reduction kernel). BandIO serves the stores of one 16-row band of a GEMM
// block: each output is a buffer resource over the band's rows that lie inside it, so stores to
// rows past M are dropped in the memory unit, and each lane's byte offset at its first column
// col0 is computed once; a column col then costs an immediate offset (col - col0 is a constant
// for all but the SwiGLU second half). The GEMM kernel loads its saved inputs itself, the same
// way (rows past M read as zero).
// epilogues that add a bias [N] (SwiGLU: [2 half], gate then up) before their activation
template <int EPI>
constexpr bool epi_has_bias() { return EPI == kEpiBf16 || EPI == kEpiGelu || EPI == kEpiSwiglu; }

struct GlobalIO {
  const GemmArgs& g;
  int64_t m;
  __device__ void load_in(int col, float (&o)[4]) const { load_bf16x4(g.aux_in, m * g.ld_in + col, o); }
  __device__ void store_c(int col, float a, float b, float c, float d) const {
    store_bf16x4(g.C, m * g.ldc + col, a, b, c, d);
  }
  __device__ void store_out(int col, float a, float b, float c, float d) const {
    store_bf16x4(g.aux_out, m * g.ld_out + col, a, b, c, d);
  }
  __device__ void store_c32(int col, f32x4 v) const {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.C) + m * g.ldc + col) = v;
  }
};

__device__ inline __amdgpu_buffer_rsrc_t band_rsrc(const void* p, int64_t ld, int esize, int row, int rows) {
  return make_rsrc(static_cast<const char*>(p) + int64_t(row) * ld * esize, uint32_t(rows * ld * esize));
}

struct BandIO {
  __amdgpu_buffer_rsrc_t c, out;
  uint32_t oc, oo;  // lane byte offsets at (band row lane % 16, column col0)
  int col0;
  __device__ void store_c(int col, float a, float b, float c_, float d) const {
    __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(a, b, c_, d), c, oc + uint32_t(col - col0) * 2, 0, 0);
  }
  __device__ void store_out(int col, float a, float b, float c_, float d) const {
    __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(a, b, c_, d), out, oo + uint32_t(col - col0) * 2, 0, 0);
  }
  __device__ void store_c32(int col, f32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), c, oc + uint32_t(col - col0) * 4, 0, 0);
  }
  // eight bf16 columns from col (16 bytes)
  __device__ void store_c16(int col, i32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, c, oc + uint32_t(col - col0) * 2, 0, 0);
  }
  __device__ void store_out16(int col, i32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, out, oo + uint32_t(col - col0) * 2, 0, 0);
  }
};

// The epilogue of one accumulator: four consecutive output columns n .. n+3 of one row, from
// x[4] = fp32 sums (SwiGLU: x = gate sums, y = up sums), the bias (if any) already added. Results:
// c -> C[., n], c2 -> C[., half + n], o -> aux_out[., n], o2 -> aux_out[., half + n], each where the
// epilogue writes it (ep_writes).
struct EpOut {
  float c[4], c2[4], o[4], o2[4];
};
enum : int { kWc = 1, kWc2 = 2, kWo = 4, kWo2 = 8 };
template <int EPI>
__device__ constexpr int ep_writes() {
  return EPI == kEpiF32 || EPI == kEpiBf16 ? kWc
       : EPI == kEpiPartialDual ? kWc | kWc2
       : EPI == kEpiGelu ? kWc | kWo
       : EPI == kEpiSwiglu ? kWc | kWo | kWo2
       : EPI == kEpiDgelu ? kWc | kWo
       : kWc | kWc2 | kWo;  // kEpiDswiglu
}

// The epilogue's saved inputs: U (GeLU gradient) or G and V (SwiGLU gradient) at columns n and
// half + n, four each.
template <int EPI>
constexpr int ep_inputs() { return EPI == kEpiDswiglu ? 2 : EPI == kEpiDgelu ? 1 : 0; }

__device__ inline void unpack_bf16x4(i32x2 v, float (&o)[4]) {
  o[0] = __uint_as_float(uint32_t(v[0]) << 16);
  o[1] = __uint_as_float(uint32_t(v[0]) & 0xffff0000u);
  o[2] = __uint_as_float(uint32_t(v[1]) << 16);
  o[3] = __uint_as_float(uint32_t(v[1]) & 0xffff0000u);
}

// Results of one accumulator from its sums and, for the gradient epilogues, the saved inputs
// u0 = aux_in[., n] and u1 = aux_in[., half + n] (already loaded).
template <int EPI>
__device__ __forceinline__ void ep_apply(const float (&x)[4], const float (&y)[4], const float (&u0)[4],
                                         const float (&u1)[4], EpOut& r) {
  if constexpr (EPI == kEpiF32 || EPI == kEpiBf16) {
    for (int v = 0; v < 4; ++v) r.c[v] = x[v];
  } else if constexpr (EPI == kEpiPartialDual) {
    for (int v = 0; v < 4; ++v) { r.c[v] = x[v]; r.c2[v] = y[v]; }
  } else if constexpr (EPI == kEpiGelu) {
    for (int v = 0; v < 4; ++v) { r.o[v] = x[v]; r.c[v] = gelu_f(x[v]); }
  } else if constexpr (EPI == kEpiSwiglu) {
    for (int v = 0; v < 4; ++v) {
      r.o[v] = x[v];
      r.o2[v] = y[v];
      r.c[v] = x[v] * sigmoid_f(x[v]) * y[v];
    }
  } else if constexpr (EPI == kEpiDgelu) {
    for (int v = 0; v < 4; ++v) {
      float d;
      gelu_and_grad(u0[v], r.o[v], d);
      r.c[v] = x[v] * d;
    }
  } else if constexpr (EPI == kEpiDswiglu) {
    for (int v = 0; v < 4; ++v) {
      const float G = u0[v], V = u1[v];
      const float sg = sigmoid_f(G);
      const float sl = G * sg;
      r.c[v] = x[v] * V * (sg * (1.0f + G * (1.0f - sg)));
      r.c2[v] = x[v] * sl;
      r.o[v] = sl * V;
    }
  }
}

template <int EPI, class IO>
__device__ __forceinline__ void ep_compute(const GemmArgs& g, const IO& io, int n, const float (&x)[4],
                                           const float (&y)[4], EpOut& r) {
  float u0[4] = {0.f, 0.f, 0.f, 0.f}, u1[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (ep_inputs<EPI>() >= 1) io.load_in(n, u0);
  if constexpr (ep_inputs<EPI>() == 2) io.load_in(int(g.half) + n, u1);
  ep_apply<EPI>(x, y, u0, u1, r);
}

// Stores of one accumulator's results, four columns (8 bytes of bf16, 16 of fp32) per lane.
template <int EPI, class IO>
__device__ __forceinline__ void ep_store4(const GemmArgs& g, const IO& io, int n, const EpOut& r) {
  constexpr int w = ep_writes<EPI>();
  if constexpr (EPI == kEpiF32 || EPI == kEpiPartialDual) {
    io.store_c32(n, f32x4{r.c[0], r.c[1], r.c[2], r.c[3]});
    if constexpr ((w & kWc2) != 0) io.store_c32(int(g.half) + n, f32x4{r.c2[0], r.c2[1], r.c2[2], r.c2[3]});
  } else {
    io.store_c(n, r.c[0], r.c[1], r.c[2], r.c[3]);
    if constexpr ((w & kWc2) != 0) io.store_c(int(g.half) + n, r.c2[0], r.c2[1], r.c2[2], r.c2[3]);
    if (g.aux_out) {
      if constexpr ((w & kWo) != 0) io.store_out(n, r.o[0], r.o[1], r.o[2], r.o[3]);
      if constexpr ((w & kWo2) != 0) io.store_out(int(g.half) + n, r.o2[0], r.o2[1], r.o2[2], r.o2[3]);
    }
  }
}

// bf16 results of two accumulators 16 columns apart (a: columns 4q..4q+3 of the first, b: of the
// second, q = lane / 16) regrouped so that each lane holds eight consecutive columns: lanes
// exchange with their neighbour 16 lanes over (v_permlane16_swap swaps the odd 16-lane rows of its
// first operand with the even rows of its second). Afterwards lane quarter q holds the first
// accumulator's columns 0..7 (q = 0), the second's 0..7 (q = 1), the first's 8..15 (q = 2) or the
// second's 8..15 (q = 3): column 16 (q & 1) + 8 (q >> 1) of the pair.
__device__ inline i32x4 pair_cols8(const float (&a)[4], const float (&b)[4]) {
  const i32x2 x = pack_bf16x4(a[0], a[1], a[2], a[3]);
  const i32x2 y = pack_bf16x4(b[0], b[1], b[2], b[3]);
  const auto s0 = __builtin_amdgcn_permlane16_swap(uint32_t(x[0]), uint32_t(y[0]), false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(uint32_t(x[1]), uint32_t(y[1]), false, false);
  return i32x4{int(s0[0]), int(s1[0]), int(s0[1]), int(s1[1])};
}

// bf16 stores of two accumulators' results (16 columns apart) as 16-byte stores, eight columns
// from n_pair per lane (pair_cols8), which gives each row 64 contiguous bytes per instruction.
// Every lane of the wave must call it (the regrouping reads other lanes); `ok` gates the stores.
template <int EPI>
__device__ __forceinline__ void ep_store_pair(const GemmArgs& g, const BandIO& io, int n_pair, bool ok,
                                              const EpOut& ra, const EpOut& rb) {
  constexpr int w = ep_writes<EPI>();
  static_assert(EPI != kEpiF32 && EPI != kEpiPartialDual, "bf16 outputs only");
  const i32x4 c = pair_cols8(ra.c, rb.c);
  if (ok) io.store_c16(n_pair, c);
  if constexpr ((w & kWc2) != 0) {
    const i32x4 c2 = pair_cols8(ra.c2, rb.c2);
    if (ok) io.store_c16(int(g.half) + n_pair, c2);
  }
  if (g.aux_out) {
    if constexpr ((w & kWo) != 0) {
      const i32x4 o = pair_cols8(ra.o, rb.o);
      if (ok) io.store_out16(n_pair, o);
    }
    if constexpr ((w & kWo2) != 0) {
      const i32x4 o2 = pair_cols8(ra.o2, rb.o2);
      if (ok) io.store_out16(int(g.half) + n_pair, o2);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------------------------- kernel
template <class TL, int LAYOUT, int EPI>
__global__ __launch_bounds__(TL::kThreads, TL::kBlocksPerCU) void gemm_kernel(GemmArgs g) {
  constexpr bool kADirect = LAYOUT != kWgrad;   // A read along k
  constexpr bool kBDirect = LAYOUT == kFwd;     // B read along k
  constexpr bool kDual = EPI == kEpiSwiglu || EPI == kEpiPartialDual;  // B tile = BN/2 gate + BN/2 up rows
  constexpr int kFM = TL::kFM, kFN = TL::kFN;
  constexpr int kOutBN = kDual ? TL::BN / 2 : TL::BN;  // output columns per block
  constexpr int kWaveN = kOutBN / TL::kWavesN;         // output columns per wave
  // the four-wave software-pipelined loop (the others: eight or four waves, one stage in flight)
  constexpr bool kPipe = TL::kWaves == 4 && TL::BM == 256;
  constexpr int kBL = kBDirect ? TL::BN : TL::kBnL;  // LDS columns of a B tile read across k
  constexpr int kStage = stage_bytes<TL, LAYOUT>();
  constexpr int kARuns = TL::kARuns, kBRuns = (kStage - TL::kATileBytes) / 1024 / TL::kWaves;
  static_assert((kADirect || TL::kNcA) && (kBDirect || TL::kNcB) && (!kDual || TL::kDualOk),
                "tile does not support this operand layout");
  static_assert(kBL == TL::BN || (kPipe && 2 * TL::BN >= kBL), "padded B tiles: pipelined loop, at least half used");

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS addresses stay scalar
  const int wm = wave / TL::kWavesN, wn = wave % TL::kWavesN;

  // ---- tile coordinates: contiguous runs per XCD, grouped order inside
  const int T = g.tiles_m * g.tiles_n;
  int tile, split;
  {
    const int G = T * g.splits;
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3, q = G >> 3, rem = G & 7;
    const int L = xcd < rem ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
    split = L / T;
    tile = L - split * T;
  }
  const int per_group = kGroupM * g.tiles_n;
  const int group = tile / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (tile % per_group) % gsz;
  const int tn = (tile % per_group) / gsz;
  const int m0 = tm * TL::BM;
  const int n0 = tn * kOutBN;

  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(g.B, g.b_bytes);

  KcLoader<kARuns> aK;
  KcLoader<kBRuns> bK;
  NcLoader<kARuns, TL::BM> aN;
  NcLoader<kBRuns, kBL> bN;
  if constexpr (kADirect) aK.init(wave, lane, g.lda, m0, g.M, false, 0, TL::BM);
  else aN.init(wave, lane, g.lda, m0, g.M, TL::BM);
  if constexpr (kBDirect) bK.init(wave, lane, g.ldb, n0, g.N, kDual, g.half, TL::BN / 2);
  else bN.init(wave, lane, g.ldb, n0, g.N, TL::BN);

  // B-tile column of fragment `in` (SwiGLU: the first half of the fragments gate, the second
  // half up, for the same output columns)
  auto bcol = [&](int in) {
    if constexpr (kDual) return (in < kFN / 2 ? 0 : TL::BN / 2) + wn * kWaveN + 16 * (in % (kFN / 2));
    else return wn * kWaveN + 16 * in;
  };
  // output column of accumulator column `in` (SwiGLU: of the gate half)
  auto ocol = [&](int in) {
    if constexpr (kDual) return n0 + wn * kWaveN + 16 * (in % (kFN / 2));
    else return n0 + wn * kWaveN + 16 * in;
  };

  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (the four-wave pipelined tiles never take accumulate = 1: the launcher checks this, since their
  // accumulators are inline-asm operands that nothing the compiler places may write late)
  if constexpr (EPI == kEpiF32 && !kPipe) {
    if (g.accumulate) {
      const float* C = reinterpret_cast<const float*>(g.C);
#pragma unroll
      for (int im = 0; im < kFM; ++im) {
        const int m = m0 + wm * TL::kWaveM + 16 * im + (lane & 15);
#pragma unroll
        for (int in = 0; in < kFN; ++in) {
          const int n = ocol(in) + 4 * (lane >> 4);
          if (m < g.M && n < g.N) acc[im][in] = *reinterpret_cast<const f32x4*>(C + int64_t(m) * g.ldc + n);
        }
      }
    }
  }

  const int nk_all = (g.K + kBK - 1) / kBK;
  // this block's run of k blocks [kb0, nk): all of them unless the product is split along k
  const int kb0 = split * g.kb_split;
  const int nk = g.splits > 1 ? min(nk_all, kb0 + g.kb_split) : nk_all;
  if constexpr (EPI == kEpiF32 || EPI == kEpiPartialDual) {
    if (g.splits > 1) g.C = reinterpret_cast<float*>(g.C) + int64_t(split) * g.part_stride;
  }

  // block-uniform: every row and column of this tile lies inside the operands
  const bool interior = (m0 + TL::BM <= g.M) && (n0 + kOutBN <= g.N);
  // Queue load runs [lo, hi) of block kb: the wave's A runs are numbered first, then its B runs.
  constexpr int kRuns = kARuns + kBRuns;
  auto issue = [&](int kb, int lo, int hi) {
    char* a_tile = smem + (kb & 1) * kStage;
    char* b_tile = a_tile + TL::kATileBytes;
    const int k0 = kb * kBK;
    const int a0 = lo < kARuns ? lo : kARuns, a1 = hi < kARuns ? hi : kARuns;
    const int b0 = lo > kARuns ? lo - kARuns : 0, b1 = hi > kARuns ? hi - kARuns : 0;
    if (interior && k0 + kBK <= g.K) {
      if (a0 < a1) {
        if constexpr (kADirect) aK.issue_fast(rsA, a_tile, wave, k0, a0, a1);
        else aN.issue_fast(rsA, a_tile, wave, k0, a0, a1);
      }
      if (b0 < b1) {
        if constexpr (kBDirect) bK.issue_fast(rsB, b_tile, wave, k0, b0, b1);
        else bN.issue_fast(rsB, b_tile, wave, k0, b0, b1);
      }
    } else {
      if (a0 < a1) {
        if constexpr (kADirect) aK.issue(rsA, a_tile, wave, k0, g.K, a0, a1);
        else aN.issue(rsA, a_tile, wave, k0, g.K, a0, a1);
      }
      if (b0 < b1) {
        if constexpr (kBDirect) bK.issue(rsB, b_tile, wave, k0, g.K, b0, b1);
        else bN.issue(rsB, b_tile, wave, k0, g.K, b0, b1);
      }
    }
  };
  auto frags = [&](int kb, bf16x8 (&af)[kFM], bf16x8 (&bf)[kFN], int kk) {
    const char* a_tile = smem + (kb & 1) * kStage;
    const char* b_tile = a_tile + TL::kATileBytes;
#pragma unroll
    for (int in = 0; in < kFN; ++in) {
      if constexpr (kBDirect) bf[in] = frag_kc(b_tile, bcol(in), lane, kk);
      else bf[in] = frag_nc<kBL>(b_tile, bcol(in), lane, kk);
    }
#pragma unroll
    for (int im = 0; im < kFM; ++im) {
      const int rbase = wm * TL::kWaveM + 16 * im;
      if constexpr (kADirect) af[im] = frag_kc(a_tile, rbase, lane, kk);
      else af[im] = frag_nc<TL::BM>(a_tile, rbase, lane, kk);
    }
  };
  auto mfmas = [&](const bf16x8 (&af)[kFM], const bf16x8 (&bf)[kFN], int im0, int im1) {
#pragma unroll
    for (int im = im0; im < im1; ++im)
#pragma unroll
      for (int in = 0; in < kFN; ++in)
        acc[im][in] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[in], af[im], acc[im][in], 0, 0, 0);
  };

  // Four-wave tiles: a software-pipelined loop for products whose K is a multiple of 64 (the
  // launcher checks this), in every operand layout and for the runs of a split product. Loads
  // skip the bounds tests: rows past M or N (columns, for an operand stored across k) read row or
  // column 0 (or zero past the operand's end) into rows and columns that the epilogue never
  // stores, and no k chunk crosses a row. With one wave per SIMD nothing else hides a wait, so the loop keeps
  // every wait off the MFMA path:
  //  - the barrier sits between the two 32-wide k steps of a block. After it, the next block's
  //    step-0 fragments are read and the loads of the block after that are issued, each between two
  //    MFMAs of step 1; step 1's own fragments are read between the MFMAs of step 0.
  //  - loads run two blocks ahead: the stage a block's loads fill was released at the barrier
  //    before (every wave had finished its reads of it), and they have a whole block to land.
  //  - the loop runs an even number of blocks; with an odd count the last one is all zeros (loads
  //    past the end read zero), and adding +0 to an fp32 sum that started at +0 changes no bit.
  //  - the LDS fragment addresses depend only on the lane, the wave and compile-time offsets (the
  //    KC swizzle of a row depends on its position within 16 rows), and the loop is unrolled over
  //    the two stages.
  //  - the MFMAs are inline asm: the 256 accumulators of a wave then stay in AGPRs with no copies,
  //    which the compiler's own MFMA form did not manage (it shuffled them through VGPRs). The
  //    compiler does not know their latency, so nothing it places may touch an accumulator early:
  //    the loop is entered with them zeroed long before (at least 64 instructions on gfx950) and
  //    leaves only at its bottom, and after it a fixed wait covers the MFMA write-to-read distance
  //    before every accumulator passes through an empty asm, which orders its reads after the wait.
  // Measured on gfx950 against the eight-wave tiles, with identical bits: 8192^3 1.38 -> 1.52
  // PFLOP/s (256 x 256), a 4096 x 2560 x 5120 product 0.97 -> 1.18 PFLOP/s (256 x 160 against 128
  // x 320).
  if constexpr (kPipe) {
    constexpr int kItems = kFM + kFN;  // fragment reads per k step
    constexpr int kStepM = kFM * kFN;  // MFMAs per k step
    // load runs ride one MFMA after a fragment read each; tiles with more runs than reads (a
    // padded B tile) spread them evenly over the k step instead
    constexpr bool kRunPerItem = kARuns + kBRuns <= kItems;
    static_assert(kRunPerItem || (kARuns + kBRuns - 1) * (kStepM - 1) / (kARuns + kBRuns) + 1 < kStepM,
                  "every load run has a slot in step 1");
    static_assert(2 * kItems <= kStepM, "a fragment read after every other MFMA of step 0");
    static_assert((kItems - 1) * kStepM / kItems + 1 < kStepM, "every load run has a slot in step 1");
    const int lr16 = lane & 15;
    const int lsw = ((lr16 >> 1) & 7) ^ ((lr16 & 1) << 2);  // swz_kc of any row r with r % 16 == lr16
    const uint32_t lo0 = lr16 * kRowBytes + (((lane >> 4) ^ lsw) << 4);      // k step 0
    const uint32_t lo1 = lr16 * kRowBytes + ((((lane >> 4) + 4) ^ lsw) << 4);  // k step 1
    const uint32_t a_wave = wm * TL::kWaveM * kRowBytes;
    const uint32_t b_wave = TL::kATileBytes + wn * kWaveN * kRowBytes;
    // An operand read across k ([64 k][tile columns]): the lane's first transposing read of the
    // fragment whose first column is cb in k step 0 (frag_nc's addressing). The swizzle of k rows
    // 8 (l / 16) + (l % 16) / 4 (+4, +32) is the same for all four, so a fragment's two reads and
    // the second k step sit at fixed distances; the XOR with the column chunk is per fragment.
    auto nc_off = [&](int cb, int cols) -> uint32_t {
      const int gq = lane >> 4, v = (lane & 15) >> 2, q = lane & 3;
      const int k0 = 8 * gq + v;
      const int chunk = (cb >> 3) + (q >> 1);
      return uint32_t(k0 * cols * 2 + ((chunk ^ swz_nc(k0)) << 4) + ((q & 1) << 3));
    };
    uint32_t a_nc[kADirect ? 1 : kFM], b_nc[kBDirect ? 1 : kFN];
    if constexpr (!kADirect) {
#pragma unroll
      for (int im = 0; im < kFM; ++im) a_nc[im] = nc_off(wm * TL::kWaveM + 16 * im, TL::BM);
    }
    if constexpr (!kBDirect) {
#pragma unroll
      for (int in = 0; in < kFN; ++in) b_nc[in] = TL::kATileBytes + nc_off(bcol(in), kBL);
    }
    auto read_nc = [](const char* p, int row_bytes) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * row_bytes));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, w);
    };
    const i32x4 rwA = raw_rsrc(g.A, g.a_bytes), rwB = raw_rsrc(g.B, g.b_bytes);
    const i32x4 rwA0 = raw_rsrc(g.A, 0), rwB0 = raw_rsrc(g.B, 0);
    // the wave's first load run in stage 0 (LDS byte address, wave-uniform)
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem)) + uint32_t(wave) * 1024u * kARuns);
    const uint32_t lds_wave_b = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem)) + uint32_t(wave) * 1024u * kBRuns);
    // each load run's lane offset (the k offset rides in the scalar offset)
    uint32_t a_voff[kARuns], b_voff[kBRuns];
#pragma unroll
    for (int j = 0; j < kARuns; ++j) {
      if constexpr (kADirect) a_voff[j] = aK.off[j];
      else a_voff[j] = aN.krow[j] * aN.ld_bytes + aN.col_off[j];
    }
#pragma unroll
    for (int j = 0; j < kBRuns; ++j) {
      if constexpr (kBDirect) b_voff[j] = bK.off[j];
      else b_voff[j] = bN.krow[j] * bN.ld_bytes + bN.col_off[j];
    }
    const uint32_t a_kstep = kADirect ? 2u : aN.ld_bytes;  // scalar offset per k element
    const uint32_t b_kstep = kBDirect ? 2u : bN.ld_bytes;
    bf16x8 a0[kFM], b0[kFN], a1[kFM], b1[kFN];
    // fragment read `i` of a k step, in the order the MFMAs first need them: A row 0, the B
    // columns, the other A rows
    auto item = [&](int stage, int kk, int i) {
      const char* st = smem + stage * kStage;
      const uint32_t lo = kk ? lo1 : lo0;
      bf16x8(&af)[kFM] = kk ? a1 : a0;
      bf16x8(&bf)[kFN] = kk ? b1 : b0;
      if (i == 0 || i > kFN) {
        const int im = i == 0 ? 0 : i - kFN;
        if constexpr (kADirect) af[im] = *reinterpret_cast<const bf16x8*>(st + a_wave + lo + im * 16 * kRowBytes);
        else af[im] = read_nc(st + a_nc[im] + kk * 32 * TL::BM * 2, TL::BM * 2);
      } else {
        const int in = i - 1;
        if constexpr (kBDirect)
          bf[in] = *reinterpret_cast<const bf16x8*>(st + b_wave + lo + (bcol(in) - wn * kWaveN) * kRowBytes);
        else bf[in] = read_nc(st + b_nc[in] + kk * 32 * kBL * 2, kBL * 2);
      }
    };
    // load run j of block kb into `stage` (the wave's A runs, then its B runs); blocks past the end
    // go through zero-size resources: every load reads zero and touches no memory
    // The loads of one block: the descriptors (zero-size past the end) and scalar k offsets are
    // chosen once per block; a run's LDS slot is the wave's base plus a constant.
    struct BlockLoads { i32x4 ra, rb; uint32_t sa, sb; };
    auto block_loads = [&](int kb) {
      const bool on = kb < nk;
      return BlockLoads{on ? rwA : rwA0, on ? rwB : rwB0, uint32_t(kb * kBK) * a_kstep, uint32_t(kb * kBK) * b_kstep};
    };
    auto load_run = [&](const BlockLoads& bl, int stage, auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < kARuns)
        dma16<j * 1024>(bl.ra, lds_wave + stage * kStage, a_voff[j], bl.sa);
      else
        dma16<(j - kARuns) * 1024>(bl.rb, lds_wave_b + stage * kStage + TL::kATileBytes,
                                   b_voff[j - kARuns], bl.sb);
    };
    // accumulator columns [0, kAccA) in AGPRs, the rest (wide tiles) in VGPRs
    constexpr int kAccA = kFM * kFN * 4 <= 256 ? kFN : 256 / (4 * kFM);
    auto mf = [&](int kk, int idx) {
      const int im = idx / kFN, in = idx % kFN;
      if (in < kAccA) {
        if (kk) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[im][in]) : "v"(b1[in]), "v"(a1[im]));
        else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[im][in]) : "v"(b0[in]), "v"(a0[im]));
      } else {
        if (kk) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[im][in]) : "v"(b1[in]), "v"(a1[im]));
        else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[im][in]) : "v"(b0[in]), "v"(a0[im]));
      }
    };
    auto block = [&](int kb, int stage) {
#pragma unroll
      for (int idx = 0; idx < kStepM; ++idx) {
        mf(0, idx);
        if ((idx & 1) && (idx >> 1) < kItems) item(stage, 1, idx >> 1);
      }
      wait_all_and_barrier();  // block kb+1 has landed; every wave is done with stage `stage`
      const BlockLoads bl = block_loads(kb + 2);
      static_for<0, kStepM>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        mf(1, p);
        static_for<0, kItems>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int at = i * kStepM / kItems;  // read i after MFMA `at`, load run i one MFMA later
          if constexpr (at == p) item(stage ^ 1, 0, i);
          if constexpr (kRunPerItem && at + 1 == p && i < kRuns) load_run(bl, stage, ic);
        });
        if constexpr (!kRunPerItem) {
          static_for<0, kRuns>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j * (kStepM - 1) / kRuns + 1 == p) load_run(bl, stage, jc);
          });
        }
      });
    };
    // this block's k blocks start at kb0 (a split product's run; 0 otherwise)
    {
      const BlockLoads bl = block_loads(kb0);
      static_for<0, kRuns>([&](auto jc) { load_run(bl, 0, jc); });
    }
    wait_all_and_barrier();
#pragma unroll
    for (int i = 0; i < kItems; ++i) item(0, 0, i);
    {
      const BlockLoads bl = block_loads(kb0 + 1);
      static_for<0, kRuns>([&](auto jc) { load_run(bl, 1, jc); });
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int kb = kb0;; kb += 2) {  // leaves at the bottom only
      block(kb, 0);
      block(kb + 1, 1);
      if (kb + 2 >= nk) break;
    }
    // 3 x 8 wait states cover the longest MFMA write -> VALU read distance (8-pass MFMA on gfx950)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int im = 0; im < kFM; ++im)
#pragma unroll
      for (int in = 0; in < kFN; ++in) {
        if (in < kAccA) asm volatile("" : "+a"(acc[im][in]));
        else asm volatile("" : "+v"(acc[im][in]));
      }
  } else {
    // Main loop. Block kb+1 is loaded while block kb is multiplied, its load runs placed between the
    // MFMA row groups of the first 32-wide step (pinned by scheduling barriers) so that load issue
    // overlaps MFMA work instead of stalling every wave right after the barrier.
    // The second 32-wide step's fragments are read while the first step multiplies. Where registers
    // allow (at most 32 MFMA tiles per wave): B after the first MFMA row, and each row's A registers
    // refilled as soon as that row's MFMAs are issued; otherwise B after the last row and A after the
    // step. Measured on gfx950: 2-9% over reading them after the first step.
    constexpr bool kEarlyA = kFM * kFN <= 32;
    // weight gradients (both operands through transposing reads) keep the plain order: their
    // fragment reads are twice as many, and reading them early measured 20-30% slower
    constexpr bool kEarly = LAYOUT != kWgrad;
    // Tiles that refill A early go in four row groups, loading half the A runs, half the A runs, half
    // the B runs, half the B runs after them. The wide tiles (more than 32 MFMA tiles per wave) load
    // after every row, an even share each: 1-3% faster for them, 2-5% slower for the others (gfx950).
    static_assert(kFM % 4 == 0, "four row groups per step");
    constexpr int kRowsPerGroup = kEarlyA ? kFM / 4 : 1;
    constexpr int kGroups = kFM / kRowsPerGroup;
    auto load_bound = [](int q) {
      if constexpr (kEarlyA) return q == 0 ? 0 : q == 1 ? kARuns / 2 : q == 2 ? kARuns : q == 3 ? kARuns + kBRuns / 2 : kRuns;
      else return q * kRuns / kFM;
    };
    if (nk > kb0) issue(kb0, 0, kRuns);
    for (int kb = kb0; kb < nk; ++kb) {
      wait_loads_and_barrier();
      const bool more = kb + 1 < nk;
      bf16x8 af[kFM], bf[kFN], bf1[kFN];
      frags(kb, af, bf, 0);
      const char* a_tile = smem + (kb & 1) * kStage;
      const char* b_tile = a_tile + TL::kATileBytes;
      auto read_b1 = [&]() {
  #pragma unroll
        for (int in = 0; in < kFN; ++in) {
          if constexpr (kBDirect) bf1[in] = frag_kc(b_tile, bcol(in), lane, 1);
          else bf1[in] = frag_nc<kBL>(b_tile, bcol(in), lane, 1);
        }
      };
      auto read_a1 = [&](int im0, int im1) {
  #pragma unroll
        for (int im = im0; im < im1; ++im) {
          const int rbase = wm * TL::kWaveM + 16 * im;
          if constexpr (kADirect) af[im] = frag_kc(a_tile, rbase, lane, 1);
          else af[im] = frag_nc<TL::BM>(a_tile, rbase, lane, 1);
        }
      };
  #pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        mfmas(af, bf, q * kRowsPerGroup, (q + 1) * kRowsPerGroup);
        __builtin_amdgcn_sched_barrier(0);
        if (more) issue(kb + 1, load_bound(q), load_bound(q + 1));
        if (kEarly && q == (kEarlyA ? 0 : kGroups - 1)) read_b1();
        if (kEarly && kEarlyA) read_a1(q * kRowsPerGroup, (q + 1) * kRowsPerGroup);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!kEarly) read_b1();
      if constexpr (!kEarly || !kEarlyA) read_a1(0, kFM);
      mfmas(af, bf1, 0, kFM);
    }
  }

  // ---- epilogue, straight from the accumulators: per accumulator (im, in), lane l holds columns
  // ocol(in) + 4 (l / 16) .. + 3 of the wave's band row 16 im + l % 16. Accumulators go in pairs
  // (in, in + 1): the lanes regroup their bf16 results so that each stores eight consecutive
  // columns, which gives every row 64 contiguous bytes per store instruction.
  constexpr int kEs = (EPI == kEpiF32 || EPI == kEpiPartialDual) ? 4 : 2;  // bytes per C element
  constexpr int kOutFN = kDual ? kFN / 2 : kFN;
  const int lr = lane & 15, lq = lane >> 4;
  const int col0 = ocol(0) + 4 * lq;
  const bool col_edge = n0 + kOutBN > g.N;  // block-uniform: some columns lie past N
  const uint32_t oc = uint32_t((int64_t(lr) * g.ldc + col0) * kEs);
  const uint32_t oo = uint32_t((int64_t(lr) * g.ld_out + col0) * 2);
  const uint32_t oi = uint32_t((int64_t(lr) * g.ld_in + col0) * 2);
  // fp32 outputs already store 16 bytes per lane: no pairs
  constexpr int kPaired = kEs == 2 ? kOutFN / 2 * 2 : 0;
  // The saved inputs of the gradient epilogues (U, or G and V) are loaded one band ahead: band
  // im + 1's loads go out before band im's stores. Loads issued after a band's stores would wait
  // for those stores as well (the vector memory counter completes in order), and each band would
  // pay a whole memory round trip.
  constexpr int kIns = ep_inputs<EPI>();
  i32x2 pin[2][kOutFN][2];
  auto fetch_in = [&](__amdgpu_buffer_rsrc_t rin, int buf) {
    if constexpr (kIns > 0) {
#pragma unroll
      for (int in = 0; in < kOutFN; ++in) {
        const int n = ocol(in) + 4 * lq;
        // as the stores: paired accumulators load for every lane, single ones inside N only
        const bool ok = in < kPaired || !col_edge || n < g.N;
        const i32x2 z = {0, 0};
        pin[buf][in][0] = ok ? __builtin_amdgcn_raw_buffer_load_b64(rin, oi + uint32_t(n - col0) * 2, 0, 0) : z;
        if constexpr (kIns == 2)
          pin[buf][in][1] =
              ok ? __builtin_amdgcn_raw_buffer_load_b64(rin, oi + uint32_t(int(g.half) + n - col0) * 2, 0, 0) : z;
      }
    }
  };
  // the bias of the lane's columns, read once for all bands (SwiGLU: gate in bx, up in by)
  const bool has_bias = epi_has_bias<EPI>() && g.bias != nullptr;
  float bx[kOutFN][4], by[kOutFN][4];
#pragma unroll
  for (int in = 0; in < kOutFN; ++in) {
    const int n = ocol(in) + 4 * lq;
    for (int v = 0; v < 4; ++v) bx[in][v] = by[in][v] = 0.0f;
    if (has_bias && (!col_edge || n < g.N)) {
      load_bf16x4(g.bias, n, bx[in]);
      if constexpr (kDual) load_bf16x4(g.bias, g.half + n, by[in]);
    }
  }
  fetch_in(band_rsrc(g.aux_in, g.ld_in, 2, m0 + wm * TL::kWaveM, min(16, g.M - (m0 + wm * TL::kWaveM))), 0);
#pragma unroll
  for (int im = 0; im < kFM; ++im) {
    const int row = m0 + wm * TL::kWaveM + 16 * im;
    if (row >= g.M) break;
    const int rows = min(16, g.M - row);
    // the next band's saved inputs (a band past M reads zeros through an empty descriptor). Its row
    // count is wave-uniform; the clamp compiles to a vector instruction, so it is read back into a
    // scalar register (a descriptor in vector registers costs a loop per load).
    if (im + 1 < kFM)
      fetch_in(band_rsrc(g.aux_in, g.ld_in, 2, row + 16, __builtin_amdgcn_readfirstlane(max(0, min(16, g.M - row - 16)))),
               (im + 1) & 1);
    BandIO io;
    io.c = band_rsrc(g.C, g.ldc, kEs, row, rows);
    io.out = band_rsrc(g.aux_out, g.ld_out, 2, row, rows);
    io.oc = oc;
    io.oo = oo;
    io.col0 = col0;
    // accumulator `in`'s results (a zero bias when there is none: one add instead of a select)
    auto compute = [&](int in, EpOut& r) {
      const f32x4 xv = acc[im][in];
      float x[4] = {xv[0], xv[1], xv[2], xv[3]};
      if constexpr (epi_has_bias<EPI>())
        for (int v = 0; v < 4; ++v) x[v] += bx[in][v];
      float u0[4] = {0.f, 0.f, 0.f, 0.f}, u1[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kIns >= 1) unpack_bf16x4(pin[im & 1][in][0], u0);
      if constexpr (kIns == 2) unpack_bf16x4(pin[im & 1][in][1], u1);
      if constexpr (kDual) {
        const f32x4 yv = acc[im][in + kFN / 2];
        float y[4] = {yv[0], yv[1], yv[2], yv[3]};
        if constexpr (epi_has_bias<EPI>())
          for (int v = 0; v < 4; ++v) y[v] += by[in][v];
        ep_apply<EPI>(x, y, u0, u1, r);
      } else {
        ep_apply<EPI>(x, x, u0, u1, r);
      }
    };
#pragma unroll
    for (int in = 0; in < kPaired; in += 2) {
      // every lane takes part in the regrouping; only the stores test the columns
      EpOut ra, rb;
      compute(in, ra);
      compute(in + 1, rb);
      const int np = ocol(in) + 16 * (lq & 1) + 8 * (lq >> 1);
      if constexpr (kEs == 2) ep_store_pair<EPI>(g, io, np, !col_edge || np < g.N, ra, rb);
    }
#pragma unroll
    for (int in = kPaired; in < kOutFN; ++in) {
      const int n = ocol(in) + 4 * lq;
      if (!col_edge || n < g.N) {
        EpOut r;
        compute(in, r);
        ep_store4<EPI>(g, io, n, r);
      }
    }
  }
}

// Explicit instantiations: with only implicit ones (from the launch switch) hipcc emits the host
// launch stub of the first instance alone.
#define TPS_GEMM_INSTANCES(TL)                                  \
  template __global__ void gemm_kernel<TL, kFwd, kEpiBf16>(GemmArgs);     \
  template __global__ void gemm_kernel<TL, kFwd, kEpiGelu>(GemmArgs);     \
  template __global__ void gemm_kernel<TL, kFwd, kEpiSwiglu>(GemmArgs);   \
  template __global__ void gemm_kernel<TL, kDgrad, kEpiBf16>(GemmArgs);   \
  template __global__ void gemm_kernel<TL, kDgrad, kEpiDgelu>(GemmArgs);  \
  template __global__ void gemm_kernel<TL, kDgrad, kEpiDswiglu>(GemmArgs); \
  template __global__ void gemm_kernel<TL, kWgrad, kEpiF32>(GemmArgs);    \
  template __global__ void gemm_kernel<TL, kDgrad, kEpiF32>(GemmArgs);
TPS_GEMM_INSTANCES(TileL)
TPS_GEMM_INSTANCES(TileS)
TPS_GEMM_INSTANCES(TileM)
TPS_GEMM_INSTANCES(TileT)
#undef TPS_GEMM_INSTANCES
template __global__ void gemm_kernel<TileL, kFwd, kEpiF32>(GemmArgs);
template __global__ void gemm_kernel<TileL, kFwd, kEpiPartialDual>(GemmArgs);
template __global__ void gemm_kernel<TileW, kFwd, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileW, kFwd, kEpiGelu>(GemmArgs);
template __global__ void gemm_kernel<TileN, kFwd, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileN, kFwd, kEpiGelu>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kFwd, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kFwd, kEpiGelu>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kFwd, kEpiSwiglu>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kDgrad, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kDgrad, kEpiDgelu>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kDgrad, kEpiDswiglu>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kDgrad, kEpiF32>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kWgrad, kEpiF32>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kFwd, kEpiF32>(GemmArgs);
template __global__ void gemm_kernel<TileL4, kFwd, kEpiPartialDual>(GemmArgs);
template __global__ void gemm_kernel<TileW4, kFwd, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileW4, kFwd, kEpiGelu>(GemmArgs);
template __global__ void gemm_kernel<TileH4, kFwd, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileH4, kFwd, kEpiGelu>(GemmArgs);
template __global__ void gemm_kernel<TileH4, kDgrad, kEpiBf16>(GemmArgs);
template __global__ void gemm_kernel<TileH4, kDgrad, kEpiDgelu>(GemmArgs);
template __global__ void gemm_kernel<TileG4, kFwd, kEpiSwiglu>(GemmArgs);

namespace {

// ------------------------------------------------------------------------------- column sums

__global__ __launch_bounds__(256) void colsum_partial_kernel(const unsigned short* X, int64_t ldx, int M, int N,
                                                             float* partials) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int chunk = blockIdx.y;
  if (n >= N) return;
  const int r0 = chunk * kColsumChunkRows;
  const int r1 = min(M, r0 + kColsumChunkRows);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += bf2f(X[int64_t(r) * ldx + n]);
  partials[int64_t(chunk) * N + n] = s;
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float* partials, int nchunks, int N, float* out,
                                                           int accumulate) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = accumulate ? out[n] : 0.f;
  for (int c = 0; c < nchunks; ++c) s += partials[int64_t(c) * N + n];
  out[n] = s;
}

__global__ void fence_kernel() {}

thread_local LaunchInfo g_last_launch;

template <class TL, int L, int E>
hipError_t launch_one(const GemmArgs& g, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  constexpr int kLds = lds_bytes<TL, L>();
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<TL, L, E>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return attr;
  const int grid = g.tiles_m * g.tiles_n * g.splits;
  g_last_launch = LaunchInfo{TL::BM, TL::BN, TL::kWavesM, TL::kWavesN, TL::kBlocksPerCU, L, E, grid, TL::kThreads};
  if (start || stop)
    hipExtLaunchKernelGGL((gemm_kernel<TL, L, E>), dim3(grid), dim3(TL::kThreads), kLds, s, start, stop,
                          0, g);
  else
    hipLaunchKernelGGL((gemm_kernel<TL, L, E>), dim3(grid), dim3(TL::kThreads), kLds, s, g);
  return hipGetLastError();
}

// The fp32 partial product of a split product (256 x 256 tiles; the four-wave pipelined ones when
// K is a multiple of 64 and `pipe` allows it; either gives the same bits).
template <class TL>
hipError_t launch_partial_tile(GemmArgs& g, int layout, bool dual, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop) {
  const int out_bn = dual ? TL::BN / 2 : TL::BN;
  g.tiles_m = (g.M + TL::BM - 1) / TL::BM;
  g.tiles_n = (g.N + out_bn - 1) / out_bn;
  if (dual) return launch_one<TL, kFwd, kEpiPartialDual>(g, stream, start, stop);
  switch (layout) {
    case kFwd: return launch_one<TL, kFwd, kEpiF32>(g, stream, start, stop);
    case kDgrad: return launch_one<TL, kDgrad, kEpiF32>(g, stream, start, stop);
    case kWgrad: return launch_one<TL, kWgrad, kEpiF32>(g, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_partial(GemmArgs& g, int layout, bool dual, bool pipe, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  if (pipe && g.K > 0 && g.K % 64 == 0) return launch_partial_tile<TileL4>(g, layout, dual, stream, start, stop);
  return launch_partial_tile<TileL>(g, layout, dual, stream, start, stop);
}

template <class TL>
hipError_t launch_tile(GemmArgs& g, int layout, int epi, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int out_bn = epi == kEpiSwiglu ? TL::BN / 2 : TL::BN;
  g.tiles_m = (g.M + TL::BM - 1) / TL::BM;
  g.tiles_n = (g.N + out_bn - 1) / out_bn;
  if constexpr (TL::kNcA && TL::kNcB && TL::kDualOk) {
    switch (layout * 8 + epi) {
      case kFwd * 8 + kEpiBf16: return launch_one<TL, kFwd, kEpiBf16>(g, stream, start, stop);
      case kFwd * 8 + kEpiGelu: return launch_one<TL, kFwd, kEpiGelu>(g, stream, start, stop);
      case kFwd * 8 + kEpiSwiglu: return launch_one<TL, kFwd, kEpiSwiglu>(g, stream, start, stop);
      case kDgrad * 8 + kEpiBf16: return launch_one<TL, kDgrad, kEpiBf16>(g, stream, start, stop);
      case kDgrad * 8 + kEpiDgelu: return launch_one<TL, kDgrad, kEpiDgelu>(g, stream, start, stop);
      case kDgrad * 8 + kEpiDswiglu: return launch_one<TL, kDgrad, kEpiDswiglu>(g, stream, start, stop);
      case kWgrad * 8 + kEpiF32: return launch_one<TL, kWgrad, kEpiF32>(g, stream, start, stop);
      case kDgrad * 8 + kEpiF32: return launch_one<TL, kDgrad, kEpiF32>(g, stream, start, stop);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (layout * 8 + epi) {
      case kFwd * 8 + kEpiBf16: return launch_one<TL, kFwd, kEpiBf16>(g, stream, start, stop);
      case kFwd * 8 + kEpiGelu: return launch_one<TL, kFwd, kEpiGelu>(g, stream, start, stop);
      default: return hipErrorInvalidValue;
    }
  }
}

// The four-wave pipelined tiles take products with K a multiple of 64 and no accumulation into an
// fp32 output (checked by the launcher), each tile a set of layouts and epilogues.
enum PipeSet : int {
  kPipeAll,     // 256 x 256: every layout and epilogue
  kPipeNarrow,  // 256 x 160: forward products without the SwiGLU pairing, activation gradients
                // with a bf16 or GeLU-gradient epilogue
  kPipeFwd,     // 256 x 320: forward products without the SwiGLU pairing
  kPipeGlu      // 256 x 224 (4 x 1 waves): forward SwiGLU products
};
template <class TL, int SET>
hipError_t launch_pipe(GemmArgs& g, int layout, int epi, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int out_bn = epi == kEpiSwiglu ? TL::BN / 2 : TL::BN;
  g.tiles_m = (g.M + TL::BM - 1) / TL::BM;
  g.tiles_n = (g.N + out_bn - 1) / out_bn;
  const int kind = layout * 8 + epi;
  if constexpr (SET == kPipeAll) {
    switch (kind) {
      case kFwd * 8 + kEpiBf16: return launch_one<TL, kFwd, kEpiBf16>(g, stream, start, stop);
      case kFwd * 8 + kEpiGelu: return launch_one<TL, kFwd, kEpiGelu>(g, stream, start, stop);
      case kFwd * 8 + kEpiSwiglu: return launch_one<TL, kFwd, kEpiSwiglu>(g, stream, start, stop);
      case kDgrad * 8 + kEpiBf16: return launch_one<TL, kDgrad, kEpiBf16>(g, stream, start, stop);
      case kDgrad * 8 + kEpiDgelu: return launch_one<TL, kDgrad, kEpiDgelu>(g, stream, start, stop);
      case kDgrad * 8 + kEpiDswiglu: return launch_one<TL, kDgrad, kEpiDswiglu>(g, stream, start, stop);
      case kDgrad * 8 + kEpiF32: return launch_one<TL, kDgrad, kEpiF32>(g, stream, start, stop);
      case kWgrad * 8 + kEpiF32: return launch_one<TL, kWgrad, kEpiF32>(g, stream, start, stop);
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (SET == kPipeNarrow) {
    switch (kind) {
      case kFwd * 8 + kEpiBf16: return launch_one<TL, kFwd, kEpiBf16>(g, stream, start, stop);
      case kFwd * 8 + kEpiGelu: return launch_one<TL, kFwd, kEpiGelu>(g, stream, start, stop);
      case kDgrad * 8 + kEpiBf16: return launch_one<TL, kDgrad, kEpiBf16>(g, stream, start, stop);
      case kDgrad * 8 + kEpiDgelu: return launch_one<TL, kDgrad, kEpiDgelu>(g, stream, start, stop);
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (SET == kPipeFwd) {
    switch (kind) {
      case kFwd * 8 + kEpiBf16: return launch_one<TL, kFwd, kEpiBf16>(g, stream, start, stop);
      case kFwd * 8 + kEpiGelu: return launch_one<TL, kFwd, kEpiGelu>(g, stream, start, stop);
      default: return hipErrorInvalidValue;
    }
  } else {
    if (kind == kFwd * 8 + kEpiSwiglu) return launch_one<TL, kFwd, kEpiSwiglu>(g, stream, start, stop);
    return hipErrorInvalidValue;
  }
}

// Block tiles the launcher chooses from, with their per-CU throughput relative to 256 x 256 when
// every CU is busy (measured on gfx950 on an 8192^3 product).
struct TileChoice {
  int id, bm, bn, blocks;
  bool fit_only;  // considered only when the product runs alone (see choose_tile)
  bool fwd_only;  // operands read along k only, with a bf16 or activation epilogue
  bool dgrad_ok;  // (fwd_only tiles) also activation gradients with a bf16 or GeLU-gradient epilogue
  bool glu_ok;    // takes the SwiGLU pairing
  bool glu_only;  // takes only the SwiGLU pairing
  bool pipe;      // four-wave pipelined: K a multiple of 64 only, no accumulation into fp32 outputs
  double rate;
  double rate_dgrad;  // dgrad_ok tiles: the rate on activation gradients
};
// The four-wave rates: 8192^3 (256 x 256) and a 4096 x 2560 x 5120 product (256 x 160, one round
// of tiles against 256 x 256's 160 tiles; as an activation gradient its B tile is padded in LDS
// and it loads 256 columns for 160).
constexpr TileChoice kTiles[] = {
    {kTile256x256, 256, 256, 1, false, false, false, true, false, false, 1.00, 1.00},
    {kTile128x128, 128, 128, 2, false, false, false, true, false, false, 0.70, 0.70},
    {kTile256x320, 256, 320, 1, true, true, false, false, false, false, 0.92, 0.0},
    {kTile128x320, 128, 320, 1, true, true, false, false, false, false, 0.73, 0.0},
    {kTile128x256, 128, 256, 1, true, false, false, true, false, false, 0.77, 0.77},
    {kTile128x128w8, 128, 128, 1, true, false, false, true, false, false, 0.50, 0.50},
    {kTile256x256w4, 256, 256, 1, false, false, false, true, false, true, 1.10, 1.10},
    {kTile256x160w4, 256, 160, 1, true, true, true, false, false, true, 0.83, 0.76},
    {kTile256x320w4, 256, 320, 1, true, true, false, false, false, true, 1.00, 0.0},
    {kTile256x224w4, 256, 224, 1, false, true, false, true, true, true, 1.05, 0.0},
};

bool tile_supports(const TileChoice& t, int64_t K, int layout, int epi, bool accumulate) {
  if (t.fwd_only) {
    const bool fwd = layout == kFwd && (epi == kEpiBf16 || epi == kEpiGelu || epi == kEpiSwiglu);
    const bool dgrad = t.dgrad_ok && layout == kDgrad && (epi == kEpiBf16 || epi == kEpiDgelu);
    if (!fwd && !dgrad) return false;
  }
  if (!t.glu_ok && epi == kEpiSwiglu) return false;
  if (t.glu_only && epi != kEpiSwiglu) return false;
  return !t.pipe || (K > 0 && K % 64 == 0 && !(accumulate && epi == kEpiF32));
}

uint32_t extent_bytes(int64_t rows, int64_t ld, int64_t cols) {
  // bytes from the base to the end of the last row actually used
  if (rows <= 0 || cols <= 0) return 0;
  return uint32_t(((rows - 1) * ld + cols) * 2);
}

}  // namespace

namespace {

// Estimated time of an M x N product with tile t, in units of one 256 x 256 tile's work at that
// tile's rate: whole rounds of resident blocks (256 CUs x blocks per CU), each round `blocks`
// tiles' work per CU at the tile's rate. `fill` receives the share of the block slots the product
// occupies over those rounds. When the products of two adjacent row slices share the GPU
// (`alone` false), the slots one product leaves empty run the other's blocks: the cost is half the
// rounds of two such products together.
double tile_cost(const TileChoice& t, int64_t M, int64_t N, int layout, int epi, bool alone, double* fill) {
  const int64_t bn = epi == kEpiSwiglu ? t.bn / 2 : t.bn;
  const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + bn - 1) / bn);
  const int64_t slots = int64_t(kCUs) * t.blocks;
  const int64_t rounds = (tiles + slots - 1) / slots;
  if (fill) *fill = rounds ? double(tiles) / double(rounds * slots) : 1.0;
  const double work = double(t.bm) * double(t.bn) / (256.0 * 256.0);
  const double r = alone ? double(rounds) : double((2 * tiles + slots - 1) / slots) / 2.0;
  return r * t.blocks * work / (layout == kDgrad ? t.rate_dgrad : t.rate);
}

}  // namespace

int choose_tile(int64_t M, int64_t N, int64_t K, int layout, int epi, bool alone, double* fill, bool accumulate) {
  // A product that runs alone gets the tile with the smallest estimated time, including the
  // tiles that exist to fill the last round. When products of adjacent slices share the GPU, the
  // CUs one leaves idle run the other's blocks, and two products that leave half the CUs idle
  // each fill them together. (A plan whose row slices' first product takes the four-wave 256 x 256
  // tile requests that tile for all its products; see plan.cpp.)
  int best = kTile256x256;
  double best_cost = 1e300, best_fill = 1.0;
  for (const TileChoice& t : kTiles) {
    if (!tile_supports(t, K, layout, epi, accumulate) || (t.fit_only && !alone)) continue;
    double f = 1.0;
    const double cost = tile_cost(t, M, N, layout, epi, alone, &f);
    if (cost < best_cost - 1e-9) { best_cost = cost; best = t.id; best_fill = f; }
  }
  if (fill) *fill = best_fill;
  return best;
}

hipError_t launch_gemm(GemmArgs g, int layout, int epi, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                       int tile, bool alone) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  g.splits = 1; g.kb_split = 0; g.part_stride = 0;  // split products go through launch_gemm_split
  // operand extents for the buffer range checks
  if (layout == kWgrad) g.a_bytes = extent_bytes(g.K, g.lda, g.M);
  else g.a_bytes = extent_bytes(g.M, g.lda, g.K);
  if (layout == kFwd) g.b_bytes = extent_bytes(epi == kEpiSwiglu ? g.half + g.N : g.N, g.ldb, g.K);
  else g.b_bytes = extent_bytes(g.K, g.ldb, g.N);
  if (g.K <= 0) { g.a_bytes = 0; g.b_bytes = 0; }
  if (tile != kTileAuto) {
    // a requested tile that cannot take this product falls back to the automatic choice
    bool ok = false;
    for (const TileChoice& t : kTiles)
      ok = ok || (t.id == tile && tile_supports(t, g.K, layout, epi, g.accumulate != 0));
    if (!ok) tile = kTileAuto;
  }
  if (tile == kTileAuto) tile = choose_tile(g.M, g.N, g.K, layout, epi, alone, nullptr, g.accumulate != 0);
  switch (tile) {
    case kTile128x128: return launch_tile<TileS>(g, layout, epi, stream, start, stop);
    case kTile256x320: return launch_tile<TileW>(g, layout, epi, stream, start, stop);
    case kTile128x320: return launch_tile<TileN>(g, layout, epi, stream, start, stop);
    case kTile128x256: return launch_tile<TileM>(g, layout, epi, stream, start, stop);
    case kTile128x128w8: return launch_tile<TileT>(g, layout, epi, stream, start, stop);
    case kTile256x256w4: return launch_pipe<TileL4, kPipeAll>(g, layout, epi, stream, start, stop);
    case kTile256x160w4: return launch_pipe<TileH4, kPipeNarrow>(g, layout, epi, stream, start, stop);
    case kTile256x320w4: return launch_pipe<TileW4, kPipeFwd>(g, layout, epi, stream, start, stop);
    case kTile256x224w4: return launch_pipe<TileG4, kPipeGlu>(g, layout, epi, stream, start, stop);
    default: return launch_tile<TileL>(g, layout, epi, stream, start, stop);
  }
}

namespace {

// Sum of the split partials of four consecutive outputs (in split order), then the product's
// epilogue, as the unsplit kernel would apply it. Partials are [splits][M][ldp] fp32; a SwiGLU
// product keeps gate sums in columns [0, N) and up sums in [N, 2N). N is a multiple of 8.
template <int EPI>
__global__ __launch_bounds__(256) void split_epilogue_kernel(GemmArgs g, const float* P, int splits, int64_t stride,
                                                             int64_t ldp) {
  const int64_t n4 = g.N / 4, total = int64_t(g.M) * n4;
  for (int64_t v = int64_t(blockIdx.x) * 256 + threadIdx.x; v < total; v += int64_t(gridDim.x) * 256) {
    const int64_t m = v / n4;
    const int n = int(v - m * n4) * 4;
    f32x4 xs = {0.f, 0.f, 0.f, 0.f}, ys = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI == kEpiF32) {
      if (g.accumulate) xs = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(g.C) + m * g.ldc + n);
    }
    for (int sp = 0; sp < splits; ++sp) {
      const float* row = P + sp * stride + m * ldp;
      xs += *reinterpret_cast<const f32x4*>(row + n);
      if constexpr (EPI == kEpiSwiglu) ys += *reinterpret_cast<const f32x4*>(row + g.N + n);
    }
    float x[4] = {xs[0], xs[1], xs[2], xs[3]};
    float y[4] = {ys[0], ys[1], ys[2], ys[3]};
    if constexpr (epi_has_bias<EPI>()) {
      if (g.bias) {
        float b[4];
        load_bf16x4(g.bias, n, b);
        for (int v = 0; v < 4; ++v) x[v] += b[v];
        if constexpr (EPI == kEpiSwiglu) {
          load_bf16x4(g.bias, g.half + n, b);
          for (int v = 0; v < 4; ++v) y[v] += b[v];
        }
      }
    }
    const GlobalIO io{g, m};
    EpOut r;
    ep_compute<EPI>(g, io, n, x, y, r);
    ep_store4<EPI>(g, io, n, r);
  }
}

template <int EPI>
hipError_t launch_split_epilogue(const GemmArgs& g, const float* P, int splits, int64_t stride, int64_t ldp,
                                 hipStream_t s, hipEvent_t stop) {
  const int64_t vecs = int64_t(g.M) * (g.N / 4);
  const int blocks = int(std::min<int64_t>((vecs + 255) / 256, int64_t(4) * kCUs));
  if (stop)
    hipExtLaunchKernelGGL(split_epilogue_kernel<EPI>, dim3(blocks), dim3(256), 0, s, nullptr, stop, 0, g, P,
                          splits, stride, ldp);
  else
    hipLaunchKernelGGL(split_epilogue_kernel<EPI>, dim3(blocks), dim3(256), 0, s, g, P, splits, stride, ldp);
  return hipGetLastError();
}

}  // namespace

double estimate_product_us(int64_t M, int64_t N, int64_t K, int layout, int epi, bool alone, int splits) {
  constexpr double kBlockUs = 1.9, kLaunchUs = 6.0;
  if (M <= 0 || N <= 0 || K <= 0) return 0.0;
  const int64_t nk = (K + kBK - 1) / kBK;
  if (splits > 1) {
    // split products run 256 x 256 tiles, `splits` runs each, then the reduction (SwiGLU: over
    // both halves of the B tile)
    const int64_t Nt = epi == kEpiSwiglu ? 2 * N : N;
    const int64_t T = ((M + 255) / 256) * ((Nt + 255) / 256);
    const int64_t kbs = (nk + splits - 1) / splits;
    const double red_us = double(2 * splits + 2) * double(M) * double(Nt) * 4.0 / 5e12 * 1e6;
    return double((T * splits + kCUs - 1) / kCUs) * double(kbs) * kBlockUs + red_us + 2 * kLaunchUs;
  }
  // not alone: M rows of two products side by side, each taking the tile the launcher picks for
  // M / 2 rows; the cost is their rounds together
  const int id = choose_tile(alone ? M : (M + 1) / 2, N, K, layout, epi, alone);
  for (const TileChoice& t : kTiles)
    if (t.id == id) return tile_cost(t, M, N, layout, epi, true, nullptr) * double(nk) * kBlockUs + kLaunchUs;
  return 0.0;
}

int choose_split(int64_t M, int64_t N, int64_t K) {
  // Estimated time in units of one 64-wide k block of a 256 x 256 tile (about 1.9 us at the
  // tile's per-CU rate): rounds of 256 tiles times the k blocks per split, plus the partials'
  // write and the reduction's reads and writes (2s + 2 fp32 passes over M x N at ~5 TB/s).
  const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t nk = (K + kBK - 1) / kBK;
  if (T <= 0 || nk <= 0) return 1;
  const double kBlockUs = 1.9;
  int best = 1;
  double best_cost = double((T + kCUs - 1) / kCUs) * double(nk);
  for (int sp = 2; sp <= 8; ++sp) {
    const int64_t kbs = (nk + sp - 1) / sp;
    if (kbs < 8) break;  // at least 512 of k per split
    const double red_us = double(2 * sp + 2) * double(M) * double(N) * 4.0 / 5e12 * 1e6;
    const double cost = double((T * sp + kCUs - 1) / kCUs) * double(kbs) + red_us / kBlockUs;
    if (cost < best_cost * 0.95) { best_cost = cost; best = sp; }
  }
  return best;
}

SplitChoice choose_split_tail(int64_t M, int64_t N, int64_t K) {
  // Costs in units of one 64-wide k block of a 256 x 256 tile (about 1.9 us), as choose_split.
  const int whole = choose_split(M, N, K);
  const int64_t Tm = (M + 255) / 256, Tn = (N + 255) / 256, nk = (K + kBK - 1) / kBK;
  if (Tm < 2 || Tn <= 0 || nk <= 0) return SplitChoice{whole, 0};
  const double kBlockUs = 1.9, kLaunchUs = 6.0;
  auto rounds = [](int64_t items) { return double((items + kCUs - 1) / kCUs); };
  auto red = [&](int64_t rows, int sp) { return double(2 * sp + 2) * double(rows) * double(N) * 4.0 / 5e12 * 1e6 / kBlockUs; };
  double best = whole > 1 ? rounds(Tm * Tn * whole) * double((nk + whole - 1) / whole) + red(M, whole)
                          : rounds(Tm * Tn) * double(nk);
  SplitChoice choice{whole, 0};
  for (int64_t t = 1; t < Tm; ++t) {
    const int64_t head_rows = (Tm - t) * 256, tail_rows = M - head_rows;
    const double head = rounds((Tm - t) * Tn) * double(nk);
    for (int sp = 2; sp <= 8; ++sp) {
      const int64_t kbs = (nk + sp - 1) / sp;
      if (kbs < 8) break;  // at least 512 of k per split
      const double cost = head + rounds(t * Tn * sp) * double(kbs) + red(tail_rows, sp) + kLaunchUs / kBlockUs;
      if (cost < best * 0.95) { best = cost; choice = SplitChoice{sp, tail_rows}; }
    }
  }
  return choice;
}

size_t split_partials_bytes(int64_t M, int64_t N, int splits) {
  return splits > 1 ? size_t(splits) * size_t(M) * size_t(N) * sizeof(float) : 0;
}

hipError_t launch_gemm_split(GemmArgs g, int layout, int epi, int splits, float* partials, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop, int tile, hipEvent_t gemm_stop, int64_t tail_rows) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool dual = epi == kEpiSwiglu;
  if (splits < 2 || splits > 64 || !partials || (dual && layout != kFwd)) return hipErrorInvalidValue;
  GemmArgs head{};
  if (tail_rows > 0 && tail_rows < g.M) {
    // the unsplit rows [0, M - tail_rows) and the split tail: g moves to the tail's first row
    const int64_t h = int64_t(g.M) - tail_rows;
    if (dual || h % 256 != 0) return hipErrorInvalidValue;
    head = g;
    head.M = int32_t(h);
    const size_t c_elem = epi == kEpiF32 ? sizeof(float) : 2;
    g.A = static_cast<const char*>(g.A) + (layout == kWgrad ? h : h * g.lda) * 2;
    g.C = static_cast<char*>(g.C) + h * g.ldc * int64_t(c_elem);
    if (g.aux_in) g.aux_in = static_cast<const char*>(g.aux_in) + h * g.ld_in * 2;
    if (g.aux_out) g.aux_out = static_cast<char*>(g.aux_out) + h * g.ld_out * 2;
    g.M = int32_t(tail_rows);
  }
  // operand extents for the buffer range checks (as launch_gemm)
  GemmArgs p = g;
  if (layout == kWgrad) p.a_bytes = extent_bytes(p.K, p.lda, p.M);
  else p.a_bytes = extent_bytes(p.M, p.lda, p.K);
  if (layout == kFwd) p.b_bytes = extent_bytes(dual ? p.half + p.N : p.N, p.ldb, p.K);
  else p.b_bytes = extent_bytes(p.K, p.ldb, p.N);
  if (p.K <= 0) { p.a_bytes = 0; p.b_bytes = 0; }
  const int64_t ldp = dual ? 2 * int64_t(p.N) : p.N;
  const int nk = (p.K + kBK - 1) / kBK;
  p.splits = splits;
  p.kb_split = (nk + splits - 1) / splits;
  p.part_stride = int64_t(p.M) * ldp;
  p.C = partials;
  p.ldc = ldp;
  p.half = dual ? p.N : 0;     // up sums' column in the partials; W1's up rows start at the same
  if (dual && g.half != g.N) return hipErrorInvalidValue;  // offset (SwiGLU: half = F' = N)
  p.accumulate = 0;
  p.bias = nullptr; p.aux_in = nullptr; p.aux_out = nullptr;
  const bool pipe = tile == kTileAuto || tile == kTile256x256w4;
  hipError_t e = launch_partial(p, layout, dual, pipe, stream, start, head.M > 0 ? nullptr : gemm_stop);
  if (e != hipSuccess) return e;
  if (head.M > 0) {
    // after the tail's partials, so that the last GEMM launch is the bulk of the product
    e = launch_gemm(head, layout, epi, stream, nullptr, gemm_stop, tile, true);
    if (e != hipSuccess) return e;
  }
  switch (epi) {
    case kEpiBf16: return launch_split_epilogue<kEpiBf16>(g, partials, splits, p.part_stride, ldp, stream, stop);
    case kEpiGelu: return launch_split_epilogue<kEpiGelu>(g, partials, splits, p.part_stride, ldp, stream, stop);
    case kEpiSwiglu: return launch_split_epilogue<kEpiSwiglu>(g, partials, splits, p.part_stride, ldp, stream, stop);
    case kEpiDgelu: return launch_split_epilogue<kEpiDgelu>(g, partials, splits, p.part_stride, ldp, stream, stop);
    case kEpiDswiglu:
      return launch_split_epilogue<kEpiDswiglu>(g, partials, splits, p.part_stride, ldp, stream, stop);
    case kEpiF32: return launch_split_epilogue<kEpiF32>(g, partials, splits, p.part_stride, ldp, stream, stop);
    default: return hipErrorInvalidValue;
  }
}

LaunchInfo last_launch() { return g_last_launch; }

hipError_t launch_fence(hipStream_t stream) {
  hipLaunchKernelGGL(fence_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError();
}

size_t colsum_partials_bytes(int32_t M, int32_t N) {
  const int64_t chunks = (int64_t(M) + kColsumChunkRows - 1) / kColsumChunkRows;
  return size_t(chunks) * size_t(N) * sizeof(float);
}

hipError_t launch_colsum(const void* X, int64_t ldx, int32_t M, int32_t N, float* partials, float* out,
                         int32_t accumulate, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int chunks = (M + kColsumChunkRows - 1) / kColsumChunkRows;
  const int nb = (N + 255) / 256;
  if (chunks > 0) {
    hipLaunchKernelGGL(colsum_partial_kernel, dim3(nb, chunks), dim3(256), 0, stream,
                       reinterpret_cast<const unsigned short*>(X), ldx, M, N, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colsum_final_kernel, dim3(nb), dim3(256), 0, stream, partials, chunks, N, out, accumulate);
  return hipGetLastError();
}

}  // namespace tps
