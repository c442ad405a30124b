// Causal attention core between the QKV and the output projections, forward, for gfx950.
//
// One block computes 128 query rows of one query head of one sequence (eight waves of 16 rows) and
// walks the key blocks of 128 up to the diagonal, keeping the softmax online (running row maximum
// and row sum, the output rescaled when the maximum grows): the tiled form of softmax attention
// that the FlashAttention titles in the Domino page's builds-on list describe. Per key block:
//   S = Q K^T   v_mfma_f32_16x16x32_bf16, Q fragments held in registers for the whole walk, K from
//               LDS by ds_read_b128 (rows XOR-swizzled by 16-byte chunk);
//   P = exp2(S log2(e) / sqrt(d) - m), rounded to bf16, m the row's reference maximum (kLazy
//               below); the mask zeroes keys past the query on the diagonal block;
//   O += P V    the same MFMA, P taken straight from S's accumulator layout (no LDS round trip)
//               and V read across keys with ds_read_b64_tr_b16.
// S's accumulator gives lane l the keys 16 j + 4 (l / 16) + 0..3 of tile j for row l % 16. The PV
// product takes a 32-key step from tiles 2c and 2c + 1 and lets lane l's eight k slots stand for
// keys 32c + 4 (l / 16) + 0..3 and 32c + 16 + 4 (l / 16) + 0..3; the V fragment is read for the same
// keys in the same slots, so the product is the plain sum over the step's keys.
// K and V tiles (128 keys x 128 dims bf16, 32 KB each) come in through registers (16-byte global
// loads one key block ahead, then ds_write_b128), shared by the block's eight waves. The row maximum
// is reduced over the row's four lanes with VALU lane swaps; the row sum of the bf16 P values comes
// out of one more MFMA per 32-key step, with a fragment of ones in V's place. The diagonal is the block's last key block (query and key blocks are both
// 128 rows), masked per row; its maximum is finite from its first key on.
// Measured on the Llama shard shapes (13B: 5 query and key/value heads; 70B: 8 query heads, 1
// key/value head) at 2048-token sequences: dealing the query blocks so that each XCD reads the K/V
// rows of few heads (its L2) and each workgroup takes a heavy and a light block raised 236 and 382
// TFLOP/s to 353 and 514. Four waves of two row tiles staged through registers needed 280
// registers (one block per CU, 125-207 TFLOP/s); with direct global -> LDS loads they fit in 252
// and two blocks per CU: attn_fwd_kernel2 below, taken when there are enough work items. Not
// adopted: four-wave 64-row blocks (each staging its own K and V, 190 and 264 before the dealing),
// double-buffered K/V with one barrier per key block (more registers; slower even with them capped
// for two blocks per CU), and capping this kernel at 128 registers for two blocks per CU (a few
// spills; 70B 3-6% faster, 13B 18% slower). 128-key blocks (half the barriers and
// softmax rounds of 64-key ones, twice the independent S tiles) ran 4-5% faster than 64-key ones;
// with 217 registers one block runs per CU.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn.hpp"

namespace tps {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = kAttnHeadDim;  // 128
constexpr int kWaves = 8;
constexpr int kBQ = 16 * kWaves;  // query rows per block
static_assert(kBQ == kAttnBlock, "the launcher's block size");
constexpr int kBK = 128;          // keys per block
constexpr int kRowB = kD * 2;     // bytes of one K or V row in LDS
constexpr int kThreads = 64 * kWaves;

// 16-byte chunk swizzles: K rows are read 16 rows at one chunk per quarter wave (chunk ^ row%16
// spreads them over all banks); V rows are read 16 rows x two chunks per transposing read (chunk ^
// 2 (row % 8) leaves two reads per bank group, the minimum for 512 bytes).
__device__ inline int swz_k(int row) { return row & 15; }
__device__ inline int swz_v(int row) { return (row & 7) << 1; }

// Online softmax with a lazy reference: a row keeps its reference maximum m (log2 units) until a
// key block's maximum exceeds it by more than kLazy, so most blocks neither rescale the output nor
// the row sum. P = exp2(S scale_log2 - m) then stays below 2^kLazy, and the row's log-sum-exp is
// m + log2(l) for whatever m it ended with. The decision depends only on the row's own scores, so
// every kernel that walks the same key blocks takes the same references and gets the same bits.
constexpr float kLazy = 8.0f;

// max of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes holding one S row), on VALU lane
// swaps; every lane of the group gets the same bits
__device__ inline float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Pairing of query blocks qb and nqb - 1 - qb in one workgroup (needs an even nqb and a whole number
// of pairs per XCD).
__host__ __device__ inline bool attn_paired(int nqb, int total) { return (nqb & 1) == 0 && (total & 15) == 0; }

__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char k_lds[kBK * kRowB];
  __shared__ __attribute__((aligned(16))) char v_lds[kBK * kRowB];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Work items (sequence, head, query block qb). Query blocks qb and nqb - 1 - qb together cost the
  // same (nqb + 1 key blocks), so where the item count allows, one workgroup takes such a pair,
  // the heavy block first, and every workgroup does the same work. Workgroups go to the eight XCDs
  // round robin by launch index; the pairs are dealt so that each XCD takes one contiguous run of
  // them (those of a few heads of one or two sequences), whose K/V rows stay in its own L2.
  const int nqb = a.seq_len / kBQ;
  const int total = nqb * a.q_heads * (a.tokens / a.seq_len), li = int(blockIdx.x);
  const bool paired = attn_paired(nqb, total);
#pragma clang loop unroll(disable)
  for (int it = 0; it < (paired ? 2 : 1); ++it) {
    int bh, qb;
    if (paired) {
      const int per_xcd = total >> 4;  // pairs per XCD
      const int u = (li & 7) * per_xcd + (li >> 3);
      const int half = nqb >> 1;
      bh = u / half;
      const int pi = u - bh * half;
      qb = it == 0 ? nqb - 1 - pi : pi;
    } else {
      bh = li / nqb;
      qb = nqb - 1 - (li - bh * nqb);  // heavier blocks of a head first
    }
    const int b = bh / a.q_heads, h = bh - b * a.q_heads;
    const int g = h / (a.q_heads / a.kv_heads);
    const int64_t seq0 = int64_t(b) * a.seq_len;  // first token row of the sequence
    const unsigned short* qkv = reinterpret_cast<const unsigned short*>(a.QKV);
    const int64_t ld = a.ld_qkv;
    const int64_t kcol = int64_t(a.q_heads + g) * kD, vcol = int64_t(a.q_heads + a.kv_heads + g) * kD;

    const int lr = lane & 15, lg = lane >> 4;
    const int q_row = qb * kBQ + wave * 16 + lr;  // this lane's query row within the sequence

    // Q fragments of the lane's row: dims 32 kk + 8 lg .. +7 (kept for the whole walk)
    bf16x8 qf[kD / 32];
    {
      const unsigned short* qp = qkv + (seq0 + q_row) * ld + int64_t(h) * kD + 8 * lg;
  #pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk);
    }

    f32x4 o[kD / 16];
  #pragma unroll
    for (int j = 0; j < kD / 16; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the row sum of P comes out of the PV product: one more MFMA per 32-key step with a fragment
    // of ones in V's place gives every lane its row's sum of the bf16 P values (the weights O uses)
    float m = -INFINITY;
    f32x4 lacc = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                         (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
    const float sl2 = a.scale_log2;

    // K and V chunks of a key block: each thread four 16-byte chunks of each, loaded into registers
    // one block ahead (the loads of block kb + 1 fly while block kb is multiplied)
    constexpr int kLoads = kBK * kRowB / (16 * kThreads);
    i32x4 kreg[kLoads], vreg[kLoads];
    auto fetch = [&](int kb) {
  #pragma unroll
      for (int p = 0; p < kLoads; ++p) {
        const int idx = p * kThreads + t;
        const int row = idx >> 4, ch = idx & 15;
        const int64_t grow = seq0 + int64_t(kb) * kBK + row;
        kreg[p] = *reinterpret_cast<const i32x4*>(qkv + grow * ld + kcol + ch * 8);
        vreg[p] = *reinterpret_cast<const i32x4*>(qkv + grow * ld + vcol + ch * 8);
      }
    };
    const int nkb = (qb * kBQ + kBQ - 1) / kBK + 1;
    const int first_diag = (qb * kBQ) / kBK;
    fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
      // ---- K and V tiles of this key block into LDS
      __syncthreads();  // every wave is done reading the previous tiles
  #pragma unroll
      for (int p = 0; p < kLoads; ++p) {
        const int idx = p * kThreads + t;
        const int row = idx >> 4, ch = idx & 15;
        *reinterpret_cast<i32x4*>(k_lds + row * kRowB + ((ch ^ swz_k(row)) << 4)) = kreg[p];
        *reinterpret_cast<i32x4*>(v_lds + row * kRowB + ((ch ^ swz_v(row)) << 4)) = vreg[p];
      }
      __syncthreads();
      if (kb + 1 < nkb) fetch(kb + 1);

      // ---- S = Q K^T for the wave's 16 rows x 128 keys: eight 16-key tiles
      f32x4 s[kBK / 16];
  #pragma unroll
      for (int j = 0; j < kBK / 16; ++j) {
        s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 16 * j + lr;
  #pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk) {
          const int ch = 4 * kk + lg;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_lds + krow * kRowB + ((ch ^ swz_k(krow)) << 4));
          // first operand K (rows = keys), second Q: lane l gets S[q row lr][key 16 j + 4 lg + v]
          s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], s[j], 0, 0, 0);
        }
      }

      // ---- online softmax over the block's keys (log2 units: the scale folds into the exponent's
      // fma; the maximum of the raw scores times the positive scale is the scaled maximum)
      // (the mask in a branch of its own: folded into one per-element test, it cost a compare and
      // a select per score on every key block)
      if (kb >= first_diag) {
  #pragma unroll
        for (int j = 0; j < kBK / 16; ++j)
  #pragma unroll
          for (int v = 0; v < 4; ++v)
            if (kb * kBK + 16 * j + 4 * lg + v > q_row) s[j][v] = -INFINITY;
      }
      float mx = -INFINITY;
  #pragma unroll
      for (int j = 0; j < kBK / 16; ++j)
  #pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[j][v]);
      mx = row_max4(mx) * sl2;
      const bool move = mx > m + kLazy;  // always on the first block (m = -inf)
      const float m_new = move ? mx : m;
      const float alpha = move ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;  // 0 on the first block
      bf16x8 pf[kBK / 32];
  #pragma unroll
      for (int c = 0; c < kBK / 32; ++c) {
  #pragma unroll
        for (int half = 0; half < 2; ++half)
  #pragma unroll
          for (int v = 0; v < 4; ++v)
            pf[c][4 * half + v] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[2 * c + half][v], sl2, -m_new));
      }
      m = m_new;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {  // (alpha = 1 on the other lanes)
  #pragma unroll
        for (int j = 0; j < kD / 16; ++j) o[j] *= alpha;
        lacc *= alpha;
      }

      // ---- O += P V: for each 32-key step, the V fragment of keys 32c + 4 lg + 0..3 and
      // 32c + 16 + 4 lg + 0..3 in the lane's k slots, dims 16 jd + lr
      const int vq = lane & 3, vv4 = (lane & 15) >> 2;
  #pragma unroll
      for (int c = 0; c < kBK / 32; ++c) {
        const int k0 = 32 * c + 4 * lg + vv4, k1 = k0 + 16;
  #pragma unroll
        for (int jd = 0; jd < kD / 16; ++jd) {
          const int ch = 2 * jd + (vq >> 1);  // 16-byte chunk of dims 16 jd + 4 vq .. +3
          const int bin = (vq & 1) << 3;
          const char* p0 = v_lds + k0 * kRowB + ((ch ^ swz_v(k0)) << 4) + bin;
          const char* p1 = v_lds + k1 * kRowB + ((ch ^ swz_v(k1)) << 4) + bin;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
          const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          // first operand V (rows = dims), second P: lane l gets O[q row lr][dim 16 jd + 4 lg + v]
          o[jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pf[c], o[jd], 0, 0, 0);
        }
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[c], lacc, 0, 0, 0);
      }
    }

    // ---- C = O / l (bf16), the lane's row and dims 16 jd + 4 lg .. +3; the row's log-sum-exp
    // (natural log) m + log2(l) in log2 units, for the backward pass
    const float lsum = lacc[0];
    const float inv = 1.0f / lsum;
    if (a.lse && lg == 0) a.lse[(seq0 + q_row) * a.q_heads + h] = (m + __log2f(lsum)) * 0.69314718055994531f;
    unsigned short* C = reinterpret_cast<unsigned short*>(a.C) + (seq0 + q_row) * a.ld_c + int64_t(h) * kD + 4 * lg;
  #pragma unroll
    for (int jd = 0; jd < kD / 16; ++jd) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 r = {(__bf16)(o[jd][0] * inv), (__bf16)(o[jd][1] * inv), (__bf16)(o[jd][2] * inv),
                        (__bf16)(o[jd][3] * inv)};
      *reinterpret_cast<i32x2*>(C + 16 * jd) = __builtin_bit_cast(i32x2, r);
    }
  }
}


// The same attention with four waves of 32 query rows (two 16-row tiles each) per 128-row block: each
// K and V fragment read from LDS serves twice the rows. K and V tiles come by direct global -> LDS
// loads (buffer_load_dwordx4 ... lds; lane l of a 1-KB run fetches the chunk the swizzle puts at
// its LDS slot), which keeps the staging registers free: 230 registers, two blocks per CU. Taken
// when the paired work items give at least two workgroups per CU; with fewer, most CUs would hold
// one four-wave block, which has no second wave per SIMD to hide its waits (the 13B shard's 160
// pairs: 82.5 us against the eight-wave kernel's 61.9), so the eight-wave kernel runs. Measured at
// the 70B shard (512 pairs): 110.3 us against 127.5, the same bits.
constexpr int kWaves2 = 4, kRT2 = 2;             // waves per block, row tiles per wave
constexpr int kBQ2 = 16 * kRT2 * kWaves2;          // 128 query rows per block
constexpr int kThreads2 = 64 * kWaves2;
static_assert(kBQ2 == kAttnBlock, "the launcher's block size");
typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(kThreads2, 2) void attn_fwd_kernel2(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char k_lds[kBK * kRowB];
  __shared__ __attribute__((aligned(1024))) char v_lds[kBK * kRowB];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nqb = a.seq_len / kBQ2;
  const int total = nqb * a.q_heads * int(a.tokens / a.seq_len), li = int(blockIdx.x);
  const bool pr = attn_paired(nqb, total);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.QKV), (short)0, (int)(uint32_t)(a.tokens * a.ld_qkv * 2), 0x00020000);
#pragma clang loop unroll(disable)
  for (int it = 0; it < (pr ? 2 : 1); ++it) {
    int bh, qb;
    if (pr) {
      const int per_xcd = total >> 4;
      const int u = (li & 7) * per_xcd + (li >> 3);
      const int half = nqb >> 1;
      bh = u / half;
      const int pi = u - bh * half;
      qb = it == 0 ? nqb - 1 - pi : pi;
    } else {
      bh = li / nqb;
      qb = nqb - 1 - (li - bh * nqb);
    }
    const int b = bh / a.q_heads, h = bh - b * a.q_heads;
    const int g = h / (a.q_heads / a.kv_heads);
    const int64_t seq0 = int64_t(b) * a.seq_len;
    const unsigned short* qkv = reinterpret_cast<const unsigned short*>(a.QKV);
    const int64_t ld = a.ld_qkv;
    const int64_t kcol = int64_t(a.q_heads + g) * kD, vcol = int64_t(a.q_heads + a.kv_heads + g) * kD;
    const int lr = lane & 15, lg = lane >> 4;
    int q_row[kRT2];
    bf16x8 qf[kRT2][kD / 32];
#pragma unroll
    for (int r = 0; r < kRT2; ++r) {
      q_row[r] = qb * kBQ2 + (wave * kRT2 + r) * 16 + lr;
      const unsigned short* qp = qkv + (seq0 + q_row[r]) * ld + int64_t(h) * kD + 8 * lg;
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) qf[r][kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk);
    }
    f32x4 o[kRT2][kD / 16];
#pragma unroll
    for (int r = 0; r < kRT2; ++r)
#pragma unroll
      for (int j = 0; j < kD / 16; ++j) o[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // row sums from the PV product, as in the eight-wave kernel
    float m[kRT2];
    f32x4 lacc[kRT2];
#pragma unroll
    for (int r = 0; r < kRT2; ++r) { m[r] = -INFINITY; lacc[r] = f32x4{0.f, 0.f, 0.f, 0.f}; }
    const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                         (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
    const float sl2 = a.scale_log2;
    // this thread's 8 runs (1 KB each) of the K tile and of the V tile: run q = wave * 8 + p covers
    // key rows 4q .. 4q + 3; lane l writes LDS bytes 16 l of the run, which hold row 4q + l / 16,
    // slot l % 16, i.e. logical chunk slot ^ swizzle(row)
    // (the swizzles repeat every 16 rows, i.e. every 4 runs: runs p and p + 4 share their lane
    // offsets, 16 rows apart through the scalar offset)
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = (wave * 8 + p) * 4 + (lane >> 4), slot = lane & 15;
      koff[p] = uint32_t((int64_t(row) * ld + kcol + ((slot ^ swz_k(row)) << 3)) * 2);
      voff[p] = uint32_t((int64_t(row) * ld + vcol + ((slot ^ swz_v(row)) << 3)) * 2);
    }
    const uint32_t row16 = uint32_t(16 * ld * 2);
    const int nkb = qb + 1;  // key blocks up to the diagonal (block sizes equal)
    for (int kb = 0; kb < nkb; ++kb) {
      __syncthreads();
      const uint32_t soff = uint32_t((seq0 + int64_t(kb) * kBK) * ld * 2);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint32_t so = soff + uint32_t(p >> 2) * row16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(k_lds + (wave * 8 + p) * 1024), 16, koff[p & 3], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(v_lds + (wave * 8 + p) * 1024), 16, voff[p & 3], so, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);  // (vmcnt 0)
      __syncthreads();
      f32x4 s[kRT2][kBK / 16];
#pragma unroll
      for (int j = 0; j < kBK / 16; ++j) {
#pragma unroll
        for (int r = 0; r < kRT2; ++r) s[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 16 * j + lr;
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk) {
          const int ch = 4 * kk + lg;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_lds + krow * kRowB + ((ch ^ swz_k(krow)) << 4));
#pragma unroll
          for (int r = 0; r < kRT2; ++r) s[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[r][kk], s[r][j], 0, 0, 0);
        }
      }
      const bool diag = kb == nkb - 1;
      bf16x8 pf[kRT2][kBK / 32];
      float alpha[kRT2];
      bool moved = false;
      if (diag) {  // (a branch of its own, as in the eight-wave kernel)
#pragma unroll
        for (int r = 0; r < kRT2; ++r)
#pragma unroll
          for (int j = 0; j < kBK / 16; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (kb * kBK + 16 * j + 4 * lg + v > q_row[r]) s[r][j][v] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < kRT2; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBK / 16; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[r][j][v]);
        mx = row_max4(mx) * sl2;
        const bool move = mx > m[r] + kLazy;
        const float m_new = move ? mx : m[r];
        alpha[r] = move ? __builtin_amdgcn_exp2f(m[r] - m_new) : 1.0f;
        moved = moved || move;
#pragma unroll
        for (int c = 0; c < kBK / 32; ++c)
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              pf[r][c][4 * half + v] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[r][2 * c + half][v], sl2, -m_new));
        m[r] = m_new;
      }
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {  // (alpha = 1 where a row kept its reference)
#pragma unroll
        for (int r = 0; r < kRT2; ++r) {
#pragma unroll
          for (int j = 0; j < kD / 16; ++j) o[r][j] *= alpha[r];
          lacc[r] *= alpha[r];
        }
      }
      const int vq = lane & 3, vv4 = (lane & 15) >> 2;
#pragma unroll
      for (int c = 0; c < kBK / 32; ++c) {
        const int k0 = 32 * c + 4 * lg + vv4, k1 = k0 + 16;
#pragma unroll
        for (int jd = 0; jd < kD / 16; ++jd) {
          const int ch = 2 * jd + (vq >> 1);
          const int bin = (vq & 1) << 3;
          const char* p0 = v_lds + k0 * kRowB + ((ch ^ swz_v(k0)) << 4) + bin;
          const char* p1 = v_lds + k1 * kRowB + ((ch ^ swz_v(k1)) << 4) + bin;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
          const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
          for (int r = 0; r < kRT2; ++r) o[r][jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[r][c], o[r][jd], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < kRT2; ++r) lacc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[r][c], lacc[r], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < kRT2; ++r) {
      const float lsum = lacc[r][0];
      const float inv = 1.0f / lsum;
      if (a.lse && lg == 0) a.lse[(seq0 + q_row[r]) * a.q_heads + h] = (m[r] + __log2f(lsum)) * 0.69314718055994531f;
      unsigned short* C = reinterpret_cast<unsigned short*>(a.C) + (seq0 + q_row[r]) * a.ld_c + int64_t(h) * kD + 4 * lg;
#pragma unroll
      for (int jd = 0; jd < kD / 16; ++jd) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 rr = {(__bf16)(o[r][jd][0] * inv), (__bf16)(o[r][jd][1] * inv), (__bf16)(o[r][jd][2] * inv),
                           (__bf16)(o[r][jd][3] * inv)};
        *reinterpret_cast<i32x2*>(C + 16 * jd) = __builtin_bit_cast(i32x2, rr);
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (a.tokens <= 0) return hipSuccess;
  const int nqb = a.seq_len / kBQ;
  const int total = nqb * a.q_heads * int(a.tokens / a.seq_len);
  const bool paired = attn_paired(nqb, total);
  const dim3 grid(unsigned(paired ? total / 2 : total));
  const bool four_waves = paired && total / 2 >= 2 * 256;
  if (four_waves) {
    if (start || stop)
      hipExtLaunchKernelGGL(attn_fwd_kernel2, grid, dim3(kThreads2), 0, stream, start, stop, 0, a);
    else
      hipLaunchKernelGGL(attn_fwd_kernel2, grid, dim3(kThreads2), 0, stream, a);
  } else if (start || stop) {
    hipExtLaunchKernelGGL(attn_fwd_kernel, grid, dim3(kThreads), 0, stream, start, stop, 0, a);
  } else {
    hipLaunchKernelGGL(attn_fwd_kernel, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tps
