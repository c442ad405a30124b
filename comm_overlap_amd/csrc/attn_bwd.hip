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
//                            with K read across keys.
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
  return launch(attn_bwd_dq_kernel, nseq * a.q_heads * (a.seq_len / kQBlock), kThreads, kDqLds, stream, nullptr,
                stop, a);
}

}  // namespace tps
