// MFMA issue-rate probe (gfx950): independent register-only chains of v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_32x32x16_bf16 at 1, 2 and 4 waves per SIMD, and the shader clock they run at (s_memtime
// against the 100 MHz s_memrealtime). The ceiling a GEMM kernel can reach with no memory traffic.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <algorithm>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int CH>
__global__ __launch_bounds__(256) void k16(int iters, float* out, unsigned long long* clk) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(0.001f * (threadIdx.x + i)); b[i] = (__bf16)(0.002f * i); }
  f32x4 acc[CH];
  for (int j = 0; j < CH; ++j) acc[j] = f32x4{float(j), 0.5f * j, 0.f, 1.f};
  unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a), "v"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  for (int j = 0; j < CH; ++j) asm volatile("" : "+a"(acc[j]));
  unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < CH; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) { clk[0] = t1 - t0; clk[1] = r1 - r0; }
}

template <int CH>
__global__ __launch_bounds__(256) void k32(int iters, float* out, unsigned long long* clk) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(0.001f * (threadIdx.x + i)); b[i] = (__bf16)(0.002f * i); }
  f32x16 acc[CH];
  for (int j = 0; j < CH; ++j) for (int v = 0; v < 16; ++v) acc[j][v] = float(j * 16 + v);
  unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a), "v"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  for (int j = 0; j < CH; ++j) asm volatile("" : "+a"(acc[j]));
  unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < CH; ++j) for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) { clk[0] = t1 - t0; clk[1] = r1 - r0; }
}

template <class K>
static void run(const char* name, K kern, int blocks, int iters, double flops_per_wave_iter) {
  float* out; unsigned long long* clk;
  if (hipMalloc(&out, size_t(blocks) * 256 * sizeof(float)) != hipSuccess ||
      hipMalloc(&clk, 2 * sizeof(unsigned long long)) != hipSuccess) {
    printf("allocation failed\n");
    return;
  }
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, iters / 4, out, clk);  // warm
  (void)hipDeviceSynchronize();
  std::vector<double> tf, ghz;
  for (int r = 0; r < 5; ++r) {
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, iters, out, clk);
    (void)hipEventRecord(e1, 0);
    (void)hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    unsigned long long c[2] = {0, 1};
    (void)hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost);
    const double fl = double(blocks) * 4 * iters * flops_per_wave_iter;
    tf.push_back(fl / (ms * 1e-3) / 1e12);
    ghz.push_back(double(c[0]) / double(c[1]) * 0.1);
  }
  std::sort(tf.begin(), tf.end()); std::sort(ghz.begin(), ghz.end());
  printf("%-28s blocks %5d: %.1f TFLOP/s (median of 5; min %.1f max %.1f), clock %.3f GHz (memtime/realtime)\n", name,
         blocks, tf[2], tf[0], tf[4], ghz[2]);
  (void)hipFree(out);
  (void)hipFree(clk);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
}

int main() {
  const int it = 20000;
  for (int blocks : {256, 512, 1024}) {
    run("16x16x32 x16 chains", k16<16>, blocks, it, 16.0 * 16 * 16 * 32 * 2);
    run("16x16x32 x32 chains", k16<32>, blocks, it / 2, 32.0 * 16 * 16 * 32 * 2);
    run("32x32x16 x4 chains", k32<4>, blocks, it, 4.0 * 32 * 32 * 16 * 2);
    run("32x32x16 x8 chains", k32<8>, blocks, it / 2, 8.0 * 32 * 32 * 16 * 2);
  }
  return 0;
}
