// Causal attention core, backward, for gfx950: the gradient of the tiled softmax attention of
// attn.hip, computed in tiles the way the FlashAttention titles in the Domino page's builds-on
// list describe (recompute the scores from Q, K and the forward's row log-sum-exp; never store the
// attention matrix). Three passes:
//   1. attn_bwd_pre_kernel   D[t, h] = dO[t, h] . O[t, h]  (= sum_s P dP, the softmax Jacobian's
//                            row term), fp32.
//   2. attn_bwd_dkv_kernel   one block per (sequence, query head, 128-key block), 8 waves of 16
//                            keys, walking the 64-query blocks from the diagonal to the end:
//                              S^T and dP^T by MFMA with the wave's K / V rows as register operands
//                              and Q / dO rows from LDS; P = exp2(S log2(e) / sqrt(d) - lse2) (one
//                              fma and an exp2; masked scores are set to -inf on diagonal steps),
//                              dS = P (dP - D); dV += P^T dO and dK += dS^T Q with dO and Q read
//                              across queries (ds_read_b64_tr_b16) and P, dS taken straight from the
//                              accumulator layout (the same 32-step slot mapping as the forward's
//                              P V product).
//   3. attn_bwd_dq_kernel    one block per (sequence, query head, 128-query block), 8 waves of 16
//                            queries, walking the key blocks up to the diagonal (the forward's
//                            structure): S and dP with K / V rows from LDS, dS as above, dQ += dS K
//                            with K read across keys. With enough blocks for two per CU,
//                            attn_bwd_dq_kernel2: four waves of two 16-query tiles (the same bits).
// A key/value head shared by several query heads (grouped heads) gets per-head fp32 partials of dK
// and dV, summed in head order by attn_bwd_group_kernel, so the result does not depend on timing.
// Every product is v_mfma_f32_16x16x32_bf16; P and dS are rounded to bf16 for their products.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn.hpp"

namespace tps {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = kAttnHeadDim;   // 128
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowB = kD * 2;      // bytes of one 128-dim bf16 row
constexpr int kKeyBlock = 128;     // keys per dK/dV block (8 waves x 16)
constexpr int kQStep = 64;         // queries per step of the dK/dV walk
constexpr int kQBlock = 128;       // queries per dQ block (8 waves x 16)
constexpr int kKStep = 128;        // keys per step of the dQ walk
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk swizzles of [rows][128 dims] tiles: rows read 16 at a time one chunk per quarter
// wave (chunk ^ row % 16), rows read across (chunk ^ 2 (row % 8)); a tile read both ways is kept
// twice.
__device__ inline int swz_r(int row) { return row & 15; }
__device__ inline int swz_t(int row) { return (row & 7) << 1; }

// Operand fragment of rows r0 .. r0 + 15 of a row-read tile: lane l gets
// tile[r0 + l % 16][dims 32 kk + 8 (l / 16) .. + 7].
__device__ inline bf16x8 frag_row(const char* tile, int r0, int lane, int kk) {
  const int row = r0 + (lane & 15);
  const int ch = 4 * kk + (lane >> 4);
  return *reinterpret_cast<const bf16x8*>(tile + row * kRowB + ((ch ^ swz_r(row)) << 4));
}

// Operand fragment read across rows of an across-read tile, for a 32-row step c: lane l gets, for
// dim 16 jd + l % 16, rows 32 c + 4 (l / 16) + 0..3 in slots 0..3 and 32 c + 16 + 4 (l / 16) + 0..3
// in slots 4..7 (the rows whose P or dS values the lane holds in those slots).
__device__ inline bf16x8 frag_across(const char* tile, int c, int jd, int lane) {
  const int g = lane >> 4, v4 = (lane & 15) >> 2, q = lane & 3;
  const int k0 = 32 * c + 4 * g + v4, k1 = k0 + 16;
  const int ch = 2 * jd + (q >> 1);
  const int bin = (q & 1) << 3;
  const char* p0 = tile + k0 * kRowB + ((ch ^ swz_t(k0)) << 4) + bin;
  const char* p1 = tile + k1 * kRowB + ((ch ^ swz_t(k1)) << 4) + bin;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ inline bf16x8 load8(const unsigned short* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ inline void store_bf16x4(unsigned short* p, float a, float b, float c, float d) {
  const bf16x4 r = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  *reinterpret_cast<i32x2*>(p) = __builtin_bit_cast(i32x2, r);
}

// ------------------------------------------------------------------------ 1. D = rowsum(dO O)
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(AttnBwdArgs a) {
  // 16 lanes per (token, head) row, 8 dims each; rows t * q_heads + h
  const int64_t rows = a.tokens * a.q_heads;
  const int64_t row = (int64_t(blockIdx.x) * 256 + threadIdx.x) >> 4;
  const int part = threadIdx.x & 15;
  float s = 0.0f;
  if (row < rows) {
    const int64_t t = row / a.q_heads, h = row - t * a.q_heads;
    const unsigned short* o = reinterpret_cast<const unsigned short*>(a.C) + t * a.ld_c + h * kD + 8 * part;
    const unsigned short* d = reinterpret_cast<const unsigned short*>(a.dC) + t * a.ld_c + h * kD + 8 * part;
    const bf16x8 ov = load8(o), dv = load8(d);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += float(ov[i]) * float(dv[i]);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
  if (row < rows && part == 0) a.Dq[row] = s;
}

// ----------------------------------------------------------------------------- 2. dK and dV
// LDS of the dK/dV kernel: Q and dO steps, each kept for row reads and for reads across rows,
// and the step's log-sum-exp and D values
constexpr int kDkvTile = kQStep * kRowB;
constexpr int kDkvLds = 4 * kDkvTile + 2 * kQStep * int(sizeof(float));

__global__ __launch_bounds__(kThreads) void attn_bwd_dkv_kernel(AttnBwdArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  char* q_r = smem;
  char* q_t = smem + kDkvTile;
  char* o_r = smem + 2 * kDkvTile;
  char* o_t = smem + 3 * kDkvTile;
  float* lse_s = reinterpret_cast<float*>(smem + 4 * kDkvTile);
  float* dd_s = lse_s + kQStep;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  // items (sequence, query head, key block), the key blocks that see the most queries first
  const int nbh = int(a.tokens / a.seq_len) * a.q_heads;
  const int item = int(blockIdx.x);
  const int kb = item / nbh, bh = item - kb * nbh;
  const int b = bh / a.q_heads, h = bh - b * a.q_heads;
  const int group = a.q_heads / a.kv_heads, g = h / group;
  const int64_t seq0 = int64_t(b) * a.seq_len;
  const unsigned short* qkv = reinterpret_cast<const unsigned short*>(a.QKV);
  const unsigned short* dO = reinterpret_cast<const unsigned short*>(a.dC);
  const int64_t ld = a.ld_qkv;
  const int64_t qcol = int64_t(h) * kD, kcol = int64_t(a.q_heads + g) * kD;
  const int64_t vcol = int64_t(a.q_heads + a.kv_heads + g) * kD;
  const int key0 = kb * kKeyBlock + 16 * wave;  // the wave's first key (within the sequence)

  // the wave's K and V rows as operands: lane l holds row key0 + l % 16, dims 32 kk + 8 (l / 16) ..
  bf16x8 kf[kD / 32], vf[kD / 32];
  {
    const unsigned short* kp = qkv + (seq0 + key0 + lr) * ld + kcol + 8 * lg;
    const unsigned short* vp = qkv + (seq0 + key0 + lr) * ld + vcol + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) {
      kf[kk] = load8(kp + 32 * kk);
      vf[kk] = load8(vp + 32 * kk);
    }
  }
  f32x4 dk[kD / 16], dv[kD / 16];
#pragma unroll
  for (int j = 0; j < kD / 16; ++j) dk[j] = dv[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Q and dO chunks of a query step in registers, one step ahead: 64 rows x 16 chunks, two per thread
  constexpr int kLoads = kQStep * kRowB / (16 * kThreads);
  i32x4 qreg[kLoads], oreg[kLoads];
  float lse_r = 0.0f, dd_r = 0.0f;
  auto fetch = [&](int qs) {
#pragma unroll
    for (int p = 0; p < kLoads; ++p) {
      const int idx = p * kThreads + t;
      const int row = idx >> 4, ch = idx & 15;
      const int64_t grow = seq0 + int64_t(qs) * kQStep + row;
      qreg[p] = *reinterpret_cast<const i32x4*>(qkv + grow * ld + qcol + ch * 8);
      oreg[p] = *reinterpret_cast<const i32x4*>(dO + grow * a.ld_c + qcol + ch * 8);
    }
    if (t < kQStep) {
      const int64_t grow = seq0 + int64_t(qs) * kQStep + t;
      lse_r = a.lse[grow * a.q_heads + h] * kLog2e;
      dd_r = a.Dq[grow * a.q_heads + h];
    }
  };
  const int nqs = a.seq_len / kQStep;
  const int qs0 = kb * kKeyBlock / kQStep;  // the first query step that sees these keys
  const float sl2 = a.scale_log2;
  fetch(qs0);
  for (int qs = qs0; qs < nqs; ++qs) {
    __syncthreads();  // every wave is done with the previous step's tiles
#pragma unroll
    for (int p = 0; p < kLoads; ++p) {
      const int idx = p * kThreads + t;
      const int row = idx >> 4, ch = idx & 15;
      *reinterpret_cast<i32x4*>(q_r + row * kRowB + ((ch ^ swz_r(row)) << 4)) = qreg[p];
      *reinterpret_cast<i32x4*>(q_t + row * kRowB + ((ch ^ swz_t(row)) << 4)) = qreg[p];
      *reinterpret_cast<i32x4*>(o_r + row * kRowB + ((ch ^ swz_r(row)) << 4)) = oreg[p];
      *reinterpret_cast<i32x4*>(o_t + row * kRowB + ((ch ^ swz_t(row)) << 4)) = oreg[p];
    }
    if (t < kQStep) {
      lse_s[t] = lse_r;
      dd_s[t] = dd_r;
    }
    __syncthreads();
    if (qs + 1 < nqs) fetch(qs + 1);

    // S^T and dP^T of the wave's 16 keys x 64 queries, as four 16-query tiles: lane l holds
    // query 16 jq + 4 (l / 16) + v (within the step) against key key0 + l % 16
    f32x4 s[kQStep / 16], dp[kQStep / 16];
#pragma unroll
    for (int jq = 0; jq < kQStep / 16; ++jq) {
      s[jq] = dp[jq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) {
        s[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_row(q_r, 16 * jq, lane, kk), kf[kk], s[jq], 0, 0, 0);
        dp[jq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_row(o_r, 16 * jq, lane, kk), vf[kk], dp[jq], 0, 0, 0);
      }
    }
    // P and dS, packed for the 32-query products: slot 4 half + v of step c holds query
    // 32 c + 16 half + 4 (l / 16) + v
    // the causal mask in a branch of its own (a masked score is -inf, its P zero): folded into one
    // per-element test it cost a compare and a select per score on every step
    const int key = key0 + lr;
    if (qs * kQStep < kb * kKeyBlock + kKeyBlock) {
#pragma unroll
      for (int jq = 0; jq < kQStep / 16; ++jq)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (key > qs * kQStep + 16 * jq + 4 * lg + v) s[jq][v] = -INFINITY;
    }
    bf16x8 pf[kQStep / 32], sf[kQStep / 32];
#pragma unroll
    for (int jq = 0; jq < kQStep / 16; ++jq)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int qi = 16 * jq + 4 * lg + v;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[jq][v], sl2, -lse_s[qi]));
        const float ds = p * (dp[jq][v] - dd_s[qi]);
        pf[jq >> 1][4 * (jq & 1) + v] = (__bf16)p;
        sf[jq >> 1][4 * (jq & 1) + v] = (__bf16)ds;
      }
    // dV += P^T dO, dK += dS^T Q: lane l accumulates key key0 + l % 16, dims 16 jd + 4 (l / 16) + v
#pragma unroll
    for (int c = 0; c < kQStep / 32; ++c)
#pragma unroll
      for (int jd = 0; jd < kD / 16; ++jd) {
        dv[jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_across(o_t, c, jd, lane), pf[c], dv[jd], 0, 0, 0);
        dk[jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_across(q_t, c, jd, lane), sf[c], dk[jd], 0, 0, 0);
      }
  }

  // dK (times 1 / sqrt(d)) and dV of the wave's keys: bf16 into dQKV when the key/value head has one
  // query head, else fp32 partials of this query head
  const float scale = a.scale;
  const int64_t grow = seq0 + key0 + lr;
  if (group == 1) {
    unsigned short* out = reinterpret_cast<unsigned short*>(a.dQKV) + grow * a.ld_qkv + 4 * lg;
#pragma unroll
    for (int jd = 0; jd < kD / 16; ++jd) {
      store_bf16x4(out + kcol + 16 * jd, dk[jd][0] * scale, dk[jd][1] * scale, dk[jd][2] * scale, dk[jd][3] * scale);
      store_bf16x4(out + vcol + 16 * jd, dv[jd][0], dv[jd][1], dv[jd][2], dv[jd][3]);
    }
  } else {
    float* pk = a.part + (int64_t(h) * a.tokens + grow) * kD + 4 * lg;
    float* pv = pk + int64_t(a.q_heads) * a.tokens * kD;
#pragma unroll
    for (int jd = 0; jd < kD / 16; ++jd) {
      *reinterpret_cast<f32x4*>(pk + 16 * jd) = dk[jd] * scale;
      *reinterpret_cast<f32x4*>(pv + 16 * jd) = dv[jd];
    }
  }
}

// Grouped heads: dK and dV of each key/value head = the sum of its query heads' partials, in head
// order. One thread per (token, key/value head, four dims).
__global__ __launch_bounds__(256) void attn_bwd_group_kernel(AttnBwdArgs a) {
  const int64_t n = a.tokens * a.kv_heads * (kD / 4);
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int d4 = int(i % (kD / 4));
  const int64_t tg = i / (kD / 4);
  const int g = int(tg % a.kv_heads);
  const int64_t tok = tg / a.kv_heads;
  const int group = a.q_heads / a.kv_heads;
  const int64_t plane = a.tokens * kD;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < group; ++j) {
    const int64_t off = (int64_t(g * group + j) * a.tokens + tok) * kD + 4 * d4;
    sk += *reinterpret_cast<const f32x4*>(a.part + off);
    sv += *reinterpret_cast<const f32x4*>(a.part + int64_t(a.q_heads) * plane + off);
  }
  unsigned short* out = reinterpret_cast<unsigned short*>(a.dQKV) + tok * a.ld_qkv + 4 * d4;
  store_bf16x4(out + int64_t(a.q_heads + g) * kD, sk[0], sk[1], sk[2], sk[3]);
  store_bf16x4(out + int64_t(a.q_heads + a.kv_heads + g) * kD, sv[0], sv[1], sv[2], sv[3]);
}

// ------------------------------------------------------------------------------------- 3. dQ
// LDS of the dQ kernel: K for row reads and for reads across keys, V for row reads
constexpr int kDqTile = kKStep * kRowB;
constexpr int kDqLds = 3 * kDqTile;

__global__ __launch_bounds__(kThreads) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  char* k_r = smem;
  char* k_t = smem + kDqTile;
  char* v_r = smem + 2 * kDqTile;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  // items (sequence, query head, query block), the blocks with the most keys first
  const int nqb = a.seq_len / kQBlock;
  const int nbh = int(a.tokens / a.seq_len) * a.q_heads;
  const int item = int(blockIdx.x);
  const int r = item / nbh, bh = item - r * nbh;
  const int qb = nqb - 1 - r;
  const int b = bh / a.q_heads, h = bh - b * a.q_heads;
  const int g = h / (a.q_heads / a.kv_heads);
  const int64_t seq0 = int64_t(b) * a.seq_len;
  const unsigned short* qkv = reinterpret_cast<const unsigned short*>(a.QKV);
  const unsigned short* dO = reinterpret_cast<const unsigned short*>(a.dC);
  const int64_t ld = a.ld_qkv;
  const int64_t qcol = int64_t(h) * kD, kcol = int64_t(a.q_heads + g) * kD;
  const int64_t vcol = int64_t(a.q_heads + a.kv_heads + g) * kD;
  const int q_row = qb * kQBlock + 16 * wave + lr;  // the lane's query (within the sequence)

  // the lane's Q and dO rows as operands (dims 32 kk + 8 (l / 16) ..), its log-sum-exp and D
  bf16x8 qf[kD / 32], of[kD / 32];
  {
    const unsigned short* qp = qkv + (seq0 + q_row) * ld + qcol + 8 * lg;
    const unsigned short* op = dO + (seq0 + q_row) * a.ld_c + qcol + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) {
      qf[kk] = load8(qp + 32 * kk);
      of[kk] = load8(op + 32 * kk);
    }
  }
  const float lse2 = a.lse[(seq0 + q_row) * a.q_heads + h] * kLog2e;
  const float dd = a.Dq[(seq0 + q_row) * a.q_heads + h];
  f32x4 dq[kD / 16];
#pragma unroll
  for (int j = 0; j < kD / 16; ++j) dq[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kLoads = kKStep * kRowB / (16 * kThreads);
  i32x4 kreg[kLoads], vreg[kLoads];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int p = 0; p < kLoads; ++p) {
      const int idx = p * kThreads + t;
      const int row = idx >> 4, ch = idx & 15;
      const int64_t grow = seq0 + int64_t(kb) * kKStep + row;
      kreg[p] = *reinterpret_cast<const i32x4*>(qkv + grow * ld + kcol + ch * 8);
      vreg[p] = *reinterpret_cast<const i32x4*>(qkv + grow * ld + vcol + ch * 8);
    }
  };
  const int nkb = (qb * kQBlock + kQBlock - 1) / kKStep + 1;
  const int first_diag = (qb * kQBlock) / kKStep;
  const float sl2 = a.scale_log2;
  fetch(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kLoads; ++p) {
      const int idx = p * kThreads + t;
      const int row = idx >> 4, ch = idx & 15;
      *reinterpret_cast<i32x4*>(k_r + row * kRowB + ((ch ^ swz_r(row)) << 4)) = kreg[p];
      *reinterpret_cast<i32x4*>(k_t + row * kRowB + ((ch ^ swz_t(row)) << 4)) = kreg[p];
      *reinterpret_cast<i32x4*>(v_r + row * kRowB + ((ch ^ swz_r(row)) << 4)) = vreg[p];
    }
    __syncthreads();
    if (kb + 1 < nkb) fetch(kb + 1);

    // S and dP of the wave's 16 queries x 128 keys: lane l holds query q_row against key
    // 16 j + 4 (l / 16) + v of the step
    f32x4 s[kKStep / 16], dp[kKStep / 16];
#pragma unroll
    for (int j = 0; j < kKStep / 16; ++j) {
      s[j] = dp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) {
        s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_row(k_r, 16 * j, lane, kk), qf[kk], s[j], 0, 0, 0);
        dp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_row(v_r, 16 * j, lane, kk), of[kk], dp[j], 0, 0, 0);
      }
    }
    if (kb >= first_diag) {  // the mask in a branch of its own, as in the dK/dV kernel
#pragma unroll
      for (int j = 0; j < kKStep / 16; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (kb * kKStep + 16 * j + 4 * lg + v > q_row) s[j][v] = -INFINITY;
    }
    bf16x8 sf[kKStep / 32];
#pragma unroll
    for (int j = 0; j < kKStep / 16; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j][v], sl2, -lse2));
        sf[j >> 1][4 * (j & 1) + v] = (__bf16)(p * (dp[j][v] - dd));
      }
    // dQ += dS K: lane l accumulates query q_row, dims 16 jd + 4 (l / 16) + v
#pragma unroll
    for (int c = 0; c < kKStep / 32; ++c)
#pragma unroll
      for (int jd = 0; jd < kD / 16; ++jd)
        dq[jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_across(k_t, c, jd, lane), sf[c], dq[jd], 0, 0, 0);
  }
  const float scale = a.scale;
  unsigned short* out = reinterpret_cast<unsigned short*>(a.dQKV) + (seq0 + q_row) * a.ld_qkv + qcol + 4 * lg;
#pragma unroll
  for (int jd = 0; jd < kD / 16; ++jd)
    store_bf16x4(out + 16 * jd, dq[jd][0] * scale, dq[jd][1] * scale, dq[jd][2] * scale, dq[jd][3] * scale);
}

// ------------------------------------------------------- 3b. dQ with four waves of two query tiles
// The same dQ with four waves of two 16-query tiles each (128 queries per block) walking 64-key
// steps: each K or V fragment read from LDS serves both tiles, half the LDS reads per MFMA of
// attn_bwd_dq_kernel, and K and V come by direct global -> LDS loads (one 1-KB run per load; lane l
// fetches the chunk the swizzle puts at its slot), so 48 KB of LDS and two blocks per CU. Every dQ
// element sums the same 32-key chunks in the same order as attn_bwd_dq_kernel, and S, P and dS are
// the same expressions: the same bits. Taken when the work items give two blocks per CU.
constexpr int kWaves2 = 4, kRT2 = 2, kThreads2 = 64 * kWaves2;
constexpr int kKStep2 = 64;                  // keys per step
constexpr int kDq2Tile = kKStep2 * kRowB;    // 16 KB per tile: K by rows, K across, V by rows
static_assert(16 * kRT2 * kWaves2 == kQBlock, "query rows per block");
static_assert(kDq2Tile == 16 * 1024 && kWaves2 * 4 * 1024 == kDq2Tile, "four 1-KB runs per wave and tile");

__global__ __launch_bounds__(kThreads2, 2) void attn_bwd_dq_kernel2(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char k_r[kDq2Tile];
  __shared__ __attribute__((aligned(1024))) char k_t[kDq2Tile];
  __shared__ __attribute__((aligned(1024))) char v_r[kDq2Tile];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nqb = a.seq_len / kQBlock;
  const int nbh = int(a.tokens / a.seq_len) * a.q_heads;
  const int item = int(blockIdx.x);
  const int rr = item / nbh, bh = item - rr * nbh;
  const int qb = nqb - 1 - rr;  // the blocks with the most keys first
  const int b = bh / a.q_heads, h = bh - b * a.q_heads;
  const int g = h / (a.q_heads / a.kv_heads);
  const int64_t seq0 = int64_t(b) * a.seq_len;
  const unsigned short* qkv = reinterpret_cast<const unsigned short*>(a.QKV);
  const unsigned short* dO = reinterpret_cast<const unsigned short*>(a.dC);
  const int64_t ld = a.ld_qkv;
  const int64_t qcol = int64_t(h) * kD, kcol = int64_t(a.q_heads + g) * kD;
  const int64_t vcol = int64_t(a.q_heads + a.kv_heads + g) * kD;

  // the lane's rows of the wave's two query tiles: Q and dO as operands, log-sum-exp and D
  int q_row[kRT2];
  bf16x8 qf[kRT2][kD / 32], of[kRT2][kD / 32];
  float lse2[kRT2], dd[kRT2];
#pragma unroll
  for (int r = 0; r < kRT2; ++r) {
    q_row[r] = qb * kQBlock + (wave * kRT2 + r) * 16 + lr;
    const unsigned short* qp = qkv + (seq0 + q_row[r]) * ld + qcol + 8 * lg;
    const unsigned short* op = dO + (seq0 + q_row[r]) * a.ld_c + qcol + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) {
      qf[r][kk] = load8(qp + 32 * kk);
      of[r][kk] = load8(op + 32 * kk);
    }
    lse2[r] = a.lse[(seq0 + q_row[r]) * a.q_heads + h] * kLog2e;
    dd[r] = a.Dq[(seq0 + q_row[r]) * a.q_heads + h];
  }
  f32x4 dq[kRT2][kD / 16];
#pragma unroll
  for (int r = 0; r < kRT2; ++r)
#pragma unroll
    for (int j = 0; j < kD / 16; ++j) dq[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this thread's four runs of each tile: run w * 4 + p holds key rows 4 (w * 4 + p) .. + 3 of the
  // step; lane l writes LDS bytes 16 l of the run (row 4 (w * 4 + p) + l / 16, slot l % 16), which
  // hold logical chunk slot ^ swizzle(row). Byte offsets from the step's first row; QKV spans less
  // than 4 GiB (checked by the launcher).
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.QKV), (short)0, (int)(uint32_t)(a.tokens * ld * 2), 0x00020000);
  uint32_t kro[4], kto[4], vro[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = (wave * 4 + p) * 4 + (lane >> 4), slot = lane & 15;
    kro[p] = uint32_t((int64_t(row) * ld + kcol + ((slot ^ swz_r(row)) << 3)) * 2);
    kto[p] = uint32_t((int64_t(row) * ld + kcol + ((slot ^ swz_t(row)) << 3)) * 2);
    vro[p] = uint32_t((int64_t(row) * ld + vcol + ((slot ^ swz_r(row)) << 3)) * 2);
  }
  const int nks = (qb * kQBlock + kQBlock) / kKStep2;  // key steps up to the diagonal
  const int first_diag = (qb * kQBlock) / kKStep2;
  const float sl2 = a.scale_log2;
  for (int ks = 0; ks < nks; ++ks) {
    __syncthreads();  // every wave is done with the previous step's tiles
    const uint32_t soff = uint32_t((seq0 + int64_t(ks) * kKStep2) * ld * 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int run = (wave * 4 + p) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(k_r + run), 16, kro[p], soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(k_t + run), 16, kto[p], soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(v_r + run), 16, vro[p], soff, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // (vmcnt 0)
    __syncthreads();

    // S and dP of both tiles x 64 keys; each K and V fragment serves the two tiles
    f32x4 s[kRT2][kKStep2 / 16], dp[kRT2][kKStep2 / 16];
#pragma unroll
    for (int j = 0; j < kKStep2 / 16; ++j) {
#pragma unroll
      for (int r = 0; r < kRT2; ++r) s[r][j] = dp[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) {
        const bf16x8 kf = frag_row(k_r, 16 * j, lane, kk);
        const bf16x8 vf = frag_row(v_r, 16 * j, lane, kk);
#pragma unroll
        for (int r = 0; r < kRT2; ++r) {
          s[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[r][kk], s[r][j], 0, 0, 0);
          dp[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, of[r][kk], dp[r][j], 0, 0, 0);
        }
      }
    }
    if (ks >= first_diag) {  // the causal mask, on the diagonal steps only
#pragma unroll
      for (int r = 0; r < kRT2; ++r)
#pragma unroll
        for (int j = 0; j < kKStep2 / 16; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (ks * kKStep2 + 16 * j + 4 * lg + v > q_row[r]) s[r][j][v] = -INFINITY;
    }
    bf16x8 sf[kRT2][kKStep2 / 32];
#pragma unroll
    for (int r = 0; r < kRT2; ++r)
#pragma unroll
      for (int j = 0; j < kKStep2 / 16; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r][j][v], sl2, -lse2[r]));
          sf[r][j >> 1][4 * (j & 1) + v] = (__bf16)(p * (dp[r][j][v] - dd[r]));
        }
    // dQ += dS K, the K fragment read across keys once for both tiles
#pragma unroll
    for (int c = 0; c < kKStep2 / 32; ++c)
#pragma unroll
      for (int jd = 0; jd < kD / 16; ++jd) {
        const bf16x8 kt = frag_across(k_t, c, jd, lane);
#pragma unroll
        for (int r = 0; r < kRT2; ++r) dq[r][jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, sf[r][c], dq[r][jd], 0, 0, 0);
      }
  }
  const float scale = a.scale;
#pragma unroll
  for (int r = 0; r < kRT2; ++r) {
    unsigned short* out = reinterpret_cast<unsigned short*>(a.dQKV) + (seq0 + q_row[r]) * a.ld_qkv + qcol + 4 * lg;
#pragma unroll
    for (int jd = 0; jd < kD / 16; ++jd)
      store_bf16x4(out + 16 * jd, dq[r][jd][0] * scale, dq[r][jd][1] * scale, dq[r][jd][2] * scale,
                   dq[r][jd][3] * scale);
  }
}

template <class K>
hipError_t launch(K kernel, int blocks, int threads, int lds, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                  const AttnBwdArgs& a) {
  if (blocks <= 0) return hipSuccess;
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), lds, s, start, stop, 0, a);
  else
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), lds, s, a);
  return hipGetLastError();
}

hipError_t set_lds_limits() {
  static const hipError_t e = [] {
    hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkv_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kDkvLds);
    if (r != hipSuccess) return r;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dq_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kDqLds);
  }();
  return e;
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t tokens, int32_t q_heads, int32_t kv_heads) {
  const size_t dq = size_t(tokens) * size_t(q_heads) * sizeof(float);
  const size_t part = q_heads == kv_heads ? 0 : 2 * size_t(q_heads) * size_t(tokens) * kD * sizeof(float);
  return (dq + 255) / 256 * 256 + part;
}

hipError_t launch_attn_bwd(AttnBwdArgs a, void* ws, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (a.tokens <= 0) return hipSuccess;
  const size_t dq_bytes = (size_t(a.tokens) * size_t(a.q_heads) * sizeof(float) + 255) / 256 * 256;
  a.Dq = static_cast<float*>(ws);
  a.part = a.q_heads == a.kv_heads ? nullptr : reinterpret_cast<float*>(static_cast<char*>(ws) + dq_bytes);
  hipError_t e = set_lds_limits();
  if (e != hipSuccess) return e;
  const int64_t rows = a.tokens * a.q_heads;
  const int nseq = int(a.tokens / a.seq_len);
  e = launch(attn_bwd_pre_kernel, int((rows * 16 + 255) / 256), 256, 0, stream, start, nullptr, a);
  if (e != hipSuccess) return e;
  e = launch(attn_bwd_dkv_kernel, nseq * a.q_heads * (a.seq_len / kKeyBlock), kThreads, kDkvLds, stream, nullptr,
             nullptr, a);
  if (e != hipSuccess) return e;
  if (a.part) {
    const int64_t n = a.tokens * a.kv_heads * (kD / 4);
    e = launch(attn_bwd_group_kernel, int((n + 255) / 256), 256, 0, stream, nullptr, nullptr, a);
    if (e != hipSuccess) return e;
  }
  const int items = nseq * a.q_heads * (a.seq_len / kQBlock);
  // the four-wave dQ kernel when its blocks fill two per CU (and its loads' 32-bit offsets span QKV)
  if (items >= 2 * 256 && a.tokens * a.ld_qkv * 2 < (int64_t(1) << 32))
    return launch(attn_bwd_dq_kernel2, items, kThreads2, 0, stream, nullptr, stop, a);
  return launch(attn_bwd_dq_kernel, items, kThreads, kDqLds, stream, nullptr, stop, a);
}

}  // namespace tps
