// bf16 MFMA GEMM family for gfx950 (MI355X) with fused layer epilogues.
//
// Block tile 256 x 256 x 64, 512 threads = 8 waves (two per SIMD, so one wave's waits hide under
// the other's MFMAs) in a 2 x 4 grid; each wave owns 128 x 64 outputs as 8 x 4
// v_mfma_f32_16x16x32_bf16 tiles with fp32 accumulators. Operand tiles go global -> LDS by direct
// loads (buffer_load_dwordx4 ... lds) into two LDS stages (128 KB): block k+1 loads while block k
// is multiplied. 16-byte XOR swizzles keep LDS traffic at full rate (chosen by measuring each
// candidate pattern's LDS throughput on gfx950):
//   * an operand read along k ("KC") is kept as [rows][64 k] (128-byte rows), fragments read
//     with ds_read_b128;
//   * an operand read across k ("NC", rows of k in memory) is kept as [64 k][256 cols] and its
//     fragments come from ds_read_b64_tr_b16, which transposes 16-bit elements across each
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

#include <cstdint>
#include <type_traits>

#include "gemm.hpp"

namespace tps {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 512;
constexpr int kTileBytes = 256 * kBK * 2;       // one operand tile, 16 KB
constexpr int kStageBytes = 2 * kTileBytes;     // A + B
constexpr int kStages = 131072 / kStageBytes;   // ring of LDS stages
constexpr int kLdsBytes = kStages * kStageBytes;  // 128 KB
constexpr int kLoadsPerBlock = kTileBytes / 1024 / 8 * 2;  // buffer_load ... lds per wave per k block
constexpr int kGroupM = 4;                      // tile rows per group of the tile order
constexpr uint32_t kOob = 0xFFFFF000u;          // buffer offset that reads as zero: operands are
                                                // smaller than 4 GiB - 4 KiB

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16-byte chunk swizzles, chosen by measurement on gfx950 (LDS read throughput of each candidate
// lane pattern): KC rows of 64 B (4 chunks) XOR the chunk with 2*(r1 ^ r3), which lets the
// fragment reads (16 consecutive rows per 16-lane group) run at full LDS rate, while the plain
// layout and the other simple XOR forms run at half rate; NC rows of 512 B XOR with
// (k & 3) << 1 | (k >> 3 & 1) << 3 for the transpose reads.
constexpr int kRowBytes = kBK * 2, kChunks = kBK / 8, kRowsPerRun = 1024 / kRowBytes;
__device__ inline int swz_kc(int row) {
  if constexpr (kBK == 32) return (((row >> 1) ^ (row >> 3)) & 1) << 1;
  else return ((row >> 1) & 7) ^ ((row & 1) << 2);
}
__device__ inline int swz_nc(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

__device__ inline float bf2f(unsigned short b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ inline float gelu_f(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }
__device__ inline float gelu_grad_f(float u) {
  return 0.5f * (1.0f + erff(u * 0.70710678118654752f)) + u * expf(-0.5f * u * u) * 0.39894228040143268f;
}
__device__ inline float sigmoid_f(float g) { return 1.0f / (1.0f + expf(-g)); }

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
// Each operand tile (16 KB = 16 runs of 1 KB) is filled by direct global -> LDS loads
// (buffer_load_dwordx4 ... lds): one load instruction writes 64 consecutive 16-byte LDS slots,
// lane l into slot l. Each of the 8 waves owns two runs of each tile; each lane loads the global
// chunk that belongs in its slot, so the swizzled layout comes from the choice of global address.
//   KC tile [256 rows][32 k]: run s holds rows 16s..16s+15; lane l -> row 16s + l/4, slot chunk l%4.
//   NC tile [32 k][256]     : run s holds k rows 2s, 2s+1; lane l -> k 2s + l/32, slot chunk l%32.
constexpr int kRuns = kTileBytes / 1024 / 8;  // runs per wave per operand tile

struct KcLoader {
  uint32_t off[kRuns];   // byte offset of the lane's chunk at k0 = 0
  uint32_t kel[kRuns];   // k index (element) of the lane's chunk at k0 = 0
  uint32_t valid;        // bit j: the chunk's row lies inside the operand
  __device__ void init(int wave, int lane, int64_t ld, int row0, int row_limit, bool dual, int64_t half) {
    valid = 0;
    for (int j = 0; j < kRuns; ++j) {
      const int r = (wave * kRuns + j) * kRowsPerRun + lane / kChunks;  // tile row
      const int ch = (lane % kChunks) ^ swz_kc(r);                      // logical chunk (k / 8)
      int li = r, gro;
      if (dual) {
        li = r & 127;
        gro = (r < 128) ? row0 + li : int(half) + row0 + li;
      } else {
        gro = row0 + r;
      }
      const bool ok = row0 + li < row_limit;
      off[j] = ok ? uint32_t(int64_t(gro) * ld * 2 + ch * 16) : 0u;
      kel[j] = uint32_t(ch * 8);
      valid |= uint32_t(ok) << j;
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0, int K) const {
    for (int j = 0; j < kRuns; ++j) {
      const bool ok = ((valid >> j) & 1) && int(kel[j]) + k0 < K;
      const uint32_t o = ok ? off[j] + uint32_t(k0) * 2 : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * kRuns + j) * 1024), 16, o, 0, 0, 0);
    }
  }
  // every chunk in range: k advances through the scalar offset, no per-lane arithmetic
  __device__ void issue_fast(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0) const {
    for (int j = 0; j < kRuns; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * kRuns + j) * 1024), 16, off[j],
                                               uint32_t(k0) * 2, 0, 0);
  }
};

struct NcLoader {
  uint32_t col_off[kRuns];  // byte offset of the lane's chunk within a k row
  uint32_t krow[kRuns];     // tile k row of the lane's chunk
  uint32_t valid;           // bit j: the chunk's columns lie inside the operand
  uint32_t ld_bytes;
  __device__ void init(int wave, int lane, int64_t ld, int col0, int col_limit) {
    valid = 0;
    ld_bytes = uint32_t(ld * 2);
    for (int j = 0; j < kRuns; ++j) {
      const int k = (wave * kRuns + j) * 2 + (lane >> 5);
      const int ch = (lane & 31) ^ swz_nc(k);
      const int c = col0 + ch * 8;
      const bool ok = c < col_limit;
      col_off[j] = ok ? uint32_t(c) * 2 : 0u;
      krow[j] = uint32_t(k);
      valid |= uint32_t(ok) << j;
    }
  }
  __device__ void issue(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0, int K) const {
    for (int j = 0; j < kRuns; ++j) {
      const int k = k0 + int(krow[j]);
      const bool ok = ((valid >> j) & 1) && k < K;
      const uint32_t o = ok ? uint32_t(k) * ld_bytes + col_off[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * kRuns + j) * 1024), 16, o, 0, 0, 0);
    }
  }
  __device__ void issue_fast(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int k0) const {
    for (int j = 0; j < kRuns; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + (wave * kRuns + j) * 1024), 16,
                                               krow[j] * ld_bytes + col_off[j], uint32_t(k0) * ld_bytes, 0, 0);
  }
};

// Wait until at most N of this wave's buffer loads are outstanding, then meet the other waves.
// Pinned in place (scheduling barriers) so that MFMA work is not moved across it.
template <int N>
__device__ inline void wait_loads_and_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}


// ------------------------------------------------------------------------------ fragment reads
// KC fragment: lane l gets operand[rb + l%16][8 (l/16) + 0..7].
__device__ inline bf16x8 frag_kc(const char* tile, int rb, int lane, int kk = 0) {
  const int row = rb + (lane & 15);
  const int ch = kk * 4 + (lane >> 4);
  return *reinterpret_cast<const bf16x8*>(tile + row * kRowBytes + ((ch ^ swz_kc(row)) << 4));
}

// NC fragment: same element assignment as frag_kc, from a [32 k][256] tile, cb = first column.
__device__ inline bf16x8 frag_nc(const char* tile, int cb, int lane, int kk = 0) {
  const int g = lane >> 4, v = (lane & 15) >> 2, q = lane & 3;
  const int chunk = (cb >> 3) + (q >> 1);
  const int k0 = kk * 32 + 8 * g + v;
  const int k1 = k0 + 4;
  const int byte_in = (q & 1) << 3;
  const char* p0 = tile + k0 * 512 + ((chunk ^ swz_nc(k0)) << 4) + byte_in;
  const char* p1 = tile + k1 * 512 + ((chunk ^ swz_nc(k1)) << 4) + byte_in;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

// ----------------------------------------------------------------------------------- epilogue
// Applied to four consecutive output columns (n .. n+3) of row m, values x[4] = fp32 sums
// (SwiGLU: x = gate sums, y = up sums).
template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& g, int m, int n, const float (&x)[4],
                                          const float (&y)[4]) {
  const int64_t mr = m;
  float o[4];
  if constexpr (EPI == kEpiF32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.C) + mr * g.ldc + n) = f32x4{x[0], x[1], x[2], x[3]};
  } else if constexpr (EPI == kEpiBf16) {
    for (int v = 0; v < 4; ++v) o[v] = x[v];
    if (g.bias) {
      float b[4];
      load_bf16x4(g.bias, n, b);
      for (int v = 0; v < 4; ++v) o[v] += b[v];
    }
    store_bf16x4(g.C, mr * g.ldc + n, o[0], o[1], o[2], o[3]);
  } else if constexpr (EPI == kEpiGelu) {
    for (int v = 0; v < 4; ++v) o[v] = x[v];
    if (g.bias) {
      float b[4];
      load_bf16x4(g.bias, n, b);
      for (int v = 0; v < 4; ++v) o[v] += b[v];
    }
    if (g.aux_out) store_bf16x4(g.aux_out, mr * g.ld_out + n, o[0], o[1], o[2], o[3]);
    for (int v = 0; v < 4; ++v) o[v] = gelu_f(o[v]);
    store_bf16x4(g.C, mr * g.ldc + n, o[0], o[1], o[2], o[3]);
  } else if constexpr (EPI == kEpiSwiglu) {
    float G[4], V[4];
    for (int v = 0; v < 4; ++v) { G[v] = x[v]; V[v] = y[v]; }
    if (g.bias) {
      float bg[4], bu[4];
      load_bf16x4(g.bias, n, bg);
      load_bf16x4(g.bias, g.half + n, bu);
      for (int v = 0; v < 4; ++v) { G[v] += bg[v]; V[v] += bu[v]; }
    }
    if (g.aux_out) {
      store_bf16x4(g.aux_out, mr * g.ld_out + n, G[0], G[1], G[2], G[3]);
      store_bf16x4(g.aux_out, mr * g.ld_out + g.half + n, V[0], V[1], V[2], V[3]);
    }
    for (int v = 0; v < 4; ++v) o[v] = G[v] * sigmoid_f(G[v]) * V[v];
    store_bf16x4(g.C, mr * g.ldc + n, o[0], o[1], o[2], o[3]);
  } else if constexpr (EPI == kEpiDgelu) {
    float u[4], h[4];
    load_bf16x4(g.aux_in, mr * g.ld_in + n, u);
    for (int v = 0; v < 4; ++v) { o[v] = x[v] * gelu_grad_f(u[v]); h[v] = gelu_f(u[v]); }
    store_bf16x4(g.C, mr * g.ldc + n, o[0], o[1], o[2], o[3]);
    store_bf16x4(g.aux_out, mr * g.ld_out + n, h[0], h[1], h[2], h[3]);
  } else if constexpr (EPI == kEpiDswiglu) {
    float G[4], V[4], dV[4], H[4];
    load_bf16x4(g.aux_in, mr * g.ld_in + n, G);
    load_bf16x4(g.aux_in, mr * g.ld_in + g.half + n, V);
    for (int v = 0; v < 4; ++v) {
      const float s = sigmoid_f(G[v]);
      const float sl = G[v] * s;
      o[v] = x[v] * V[v] * (s * (1.0f + G[v] * (1.0f - s)));
      dV[v] = x[v] * sl;
      H[v] = sl * V[v];
    }
    store_bf16x4(g.C, mr * g.ldc + n, o[0], o[1], o[2], o[3]);
    store_bf16x4(g.C, mr * g.ldc + g.half + n, dV[0], dV[1], dV[2], dV[3]);
    store_bf16x4(g.aux_out, mr * g.ld_out + n, H[0], H[1], H[2], H[3]);
  }
}

// ------------------------------------------------------------------------------------- kernel
// 8 waves (2 per SIMD, so one wave's waits hide under the other's MFMAs) in a 2 (m) x 4 (n) grid;
// wave tile 128 x 64 = 8 x 4 MFMA tiles, 128 fp32 accumulators per lane.
constexpr int kWavesN = 4;
constexpr int kFM = 8, kFN = 4;  // MFMA tiles per wave along m and n

template <int LAYOUT, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g) {
  constexpr bool kADirect = LAYOUT != kWgrad;   // A read along k
  constexpr bool kBDirect = LAYOUT == kFwd;     // B read along k
  constexpr bool kDual = EPI == kEpiSwiglu;     // B tile = 128 gate rows + 128 up rows
  constexpr int kOutBN = kDual ? kBN / 2 : kBN; // output columns per block
  constexpr int kWaveN = kOutBN / kWavesN;      // output columns per wave (64, SwiGLU 32)

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: LDS addresses stay scalar
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // ---- tile coordinates: contiguous runs per XCD, grouped order inside
  const int T = g.tiles_m * g.tiles_n;
  int tile;
  {
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3, q = T >> 3, rem = T & 7;
    tile = xcd < rem ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
  }
  const int per_group = kGroupM * g.tiles_n;
  const int group = tile / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (tile % per_group) % gsz;
  const int tn = (tile % per_group) / gsz;
  const int m0 = tm * kBM;
  const int n0 = tn * kOutBN;

  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(g.B, g.b_bytes);

  KcLoader aK, bK;
  NcLoader aN, bN;
  if constexpr (kADirect) aK.init(wave, lane, g.lda, m0, g.M, false, 0);
  else aN.init(wave, lane, g.lda, m0, g.M);
  if constexpr (kBDirect) bK.init(wave, lane, g.ldb, n0, g.N, kDual, g.half);
  else bN.init(wave, lane, g.ldb, n0, g.N);

  // B-tile column of fragment `in` (SwiGLU: fragments 0, 1 gate, 2, 3 up of the same outputs)
  auto bcol = [&](int in) {
    if constexpr (kDual) return (in < kFN / 2 ? 0 : 128) + wn * kWaveN + 16 * (in % (kFN / 2));
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

  if constexpr (EPI == kEpiF32) {
    if (g.accumulate) {
      const float* C = reinterpret_cast<const float*>(g.C);
#pragma unroll
      for (int im = 0; im < kFM; ++im) {
        const int m = m0 + wm * 128 + 16 * im + (lane & 15);
#pragma unroll
        for (int in = 0; in < kFN; ++in) {
          const int n = ocol(in) + 4 * (lane >> 4);
          if (m < g.M && n < g.N) acc[im][in] = *reinterpret_cast<const f32x4*>(C + int64_t(m) * g.ldc + n);
        }
      }
    }
  }

  const int nk = (g.K + kBK - 1) / kBK;

  // block-uniform: every row and column of this tile lies inside the operands
  const bool interior = (m0 + kBM <= g.M) && (n0 + kOutBN <= g.N);
  auto issue = [&](int kb) {
    char* a_tile = smem + (kb % kStages) * kStageBytes;
    char* b_tile = a_tile + kTileBytes;
    const int k0 = kb * kBK;
    if (interior && k0 + kBK <= g.K) {
      if constexpr (kADirect) aK.issue_fast(rsA, a_tile, wave, k0); else aN.issue_fast(rsA, a_tile, wave, k0);
      if constexpr (kBDirect) bK.issue_fast(rsB, b_tile, wave, k0); else bN.issue_fast(rsB, b_tile, wave, k0);
    } else {
      if constexpr (kADirect) aK.issue(rsA, a_tile, wave, k0, g.K); else aN.issue(rsA, a_tile, wave, k0, g.K);
      if constexpr (kBDirect) bK.issue(rsB, b_tile, wave, k0, g.K); else bN.issue(rsB, b_tile, wave, k0, g.K);
    }
  };
  auto frags = [&](int kb, bf16x8 (&af)[kFM], bf16x8 (&bf)[kFN], int kk = 0) {
    const char* a_tile = smem + (kb % kStages) * kStageBytes;
    const char* b_tile = a_tile + kTileBytes;
#pragma unroll
    for (int in = 0; in < kFN; ++in) {
      if constexpr (kBDirect) bf[in] = frag_kc(b_tile, bcol(in), lane, kk);
      else bf[in] = frag_nc(b_tile, bcol(in), lane, kk);
    }
#pragma unroll
    for (int im = 0; im < kFM; ++im) {
      const int rbase = wm * 128 + 16 * im;
      if constexpr (kADirect) af[im] = frag_kc(a_tile, rbase, lane, kk);
      else af[im] = frag_nc(a_tile, rbase, lane, kk);
    }
  };
  auto mfmas = [&](const bf16x8 (&af)[kFM], const bf16x8 (&bf)[kFN]) {
#pragma unroll
    for (int im = 0; im < kFM; ++im)
#pragma unroll
      for (int in = 0; in < kFN; ++in)
        acc[im][in] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[in], af[im], acc[im][in], 0, 0, 0);
  };
  // wait for block `kb` to land in LDS, given how many later blocks have been issued
  constexpr int kAhead = kStages - 1;
  auto wait_block = [&](int kb) {
    const int later = min(nk - 1, kb + kAhead - 1) - kb;  // blocks issued after kb
    if constexpr (kAhead >= 3) {
      if (later >= 2) { wait_loads_and_barrier<2 * kLoadsPerBlock>(); return; }
    }
    if (later >= 1) wait_loads_and_barrier<kLoadsPerBlock>();
    else wait_loads_and_barrier<0>();
  };

  if (nk > 0)
    for (int kb = 0; kb < min(nk, kAhead); ++kb) issue(kb);
  for (int kb = 0; kb < nk; ++kb) {
    wait_block(kb);
    if (kb + kAhead < nk) issue(kb + kAhead);
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      bf16x8 af[kFM], bf[kFN];
      frags(kb, af, bf, kk);
      mfmas(af, bf);
    }
  }
  __syncthreads();

  // ---- epilogue: per 16-row band, the wave parks its sums in LDS and re-reads them as whole row
  // segments, so global loads and stores of the epilogue are contiguous.
  constexpr int kEpLd = 136;  // floats per parked row (full-rate LDS writes, measured)
  float* park = reinterpret_cast<float*>(smem) + wave * 16 * kEpLd;
  const int prow = lane & 15, pcol = 4 * (lane >> 4);
#pragma unroll
  for (int im = 0; im < kFM; ++im) {
#pragma unroll
    for (int in = 0; in < kFN; ++in)
      *reinterpret_cast<f32x4*>(park + prow * kEpLd + 16 * in + pcol) = acc[im][in];
    __syncthreads();
    const int mbase = m0 + wm * 128 + 16 * im;
    // a parked row holds the wave's 64 accumulator columns (SwiGLU: 32 gate then 32 up)
    constexpr int kOutCols = kDual ? 32 : 64;
    constexpr int kLanesPerRow = kOutCols / 4;
    constexpr int kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll 1
    for (int p = 0; p < 16 / kRowsPerPass; ++p) {
      const int r = p * kRowsPerPass + lane / kLanesPerRow;
      const int c = 4 * (lane % kLanesPerRow);
      const int m = mbase + r, n = n0 + wn * kWaveN + c;
      if (m < g.M && n < g.N) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(park + r * kEpLd + c);
        const float x[4] = {xv[0], xv[1], xv[2], xv[3]};
        if constexpr (kDual) {
          const f32x4 yv = *reinterpret_cast<const f32x4*>(park + r * kEpLd + 32 + c);
          const float y[4] = {yv[0], yv[1], yv[2], yv[3]};
          epilogue4<EPI>(g, m, n, x, y);
        } else {
          epilogue4<EPI>(g, m, n, x, x);
        }
      }
    }
    __syncthreads();
  }
}

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

template <int L, int E>
hipError_t launch_one(const GemmArgs& g, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<L, E>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr != hipSuccess) return attr;
  const int grid = g.tiles_m * g.tiles_n;
  if (start || stop)
    hipExtLaunchKernelGGL((gemm_kernel<L, E>), dim3(grid), dim3(kThreads), kLdsBytes, s, start, stop, 0, g);
  else
    hipLaunchKernelGGL((gemm_kernel<L, E>), dim3(grid), dim3(kThreads), kLdsBytes, s, g);
  return hipGetLastError();
}

uint32_t extent_bytes(int64_t rows, int64_t ld, int64_t cols) {
  // bytes from the base to the end of the last row actually used
  if (rows <= 0 || cols <= 0) return 0;
  return uint32_t(((rows - 1) * ld + cols) * 2);
}

}  // namespace

hipError_t launch_gemm(GemmArgs g, int layout, int epi, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int out_bn = epi == kEpiSwiglu ? kBN / 2 : kBN;
  g.tiles_m = (g.M + kBM - 1) / kBM;
  g.tiles_n = (g.N + out_bn - 1) / out_bn;
  // operand extents for the buffer range checks
  if (layout == kWgrad) g.a_bytes = extent_bytes(g.K, g.lda, g.M);
  else g.a_bytes = extent_bytes(g.M, g.lda, g.K);
  if (layout == kFwd) g.b_bytes = extent_bytes(epi == kEpiSwiglu ? g.half + g.N : g.N, g.ldb, g.K);
  else g.b_bytes = extent_bytes(g.K, g.ldb, g.N);
  if (g.K <= 0) { g.a_bytes = 0; g.b_bytes = 0; }
  switch (layout * 8 + epi) {
    case kFwd * 8 + kEpiBf16: return launch_one<kFwd, kEpiBf16>(g, stream, start, stop);
    case kFwd * 8 + kEpiGelu: return launch_one<kFwd, kEpiGelu>(g, stream, start, stop);
    case kFwd * 8 + kEpiSwiglu: return launch_one<kFwd, kEpiSwiglu>(g, stream, start, stop);
    case kDgrad * 8 + kEpiBf16: return launch_one<kDgrad, kEpiBf16>(g, stream, start, stop);
    case kDgrad * 8 + kEpiDgelu: return launch_one<kDgrad, kEpiDgelu>(g, stream, start, stop);
    case kDgrad * 8 + kEpiDswiglu: return launch_one<kDgrad, kEpiDswiglu>(g, stream, start, stop);
    case kWgrad * 8 + kEpiF32: return launch_one<kWgrad, kEpiF32>(g, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

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
