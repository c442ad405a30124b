// Counter probe of the four-wave 256 x 256 GEMM kernel: one product of the Llama-3 70B MLP dX shape
// over all tokens (M 16384 x N 8192 x K 7168, bf16 operands filled from a seeded hash), launched 12
// times through the library's own launcher. Argument 'fwd': both operands read along k; otherwise
// the activation-gradient layout (B read across k). Run under rocprofv3 --pmc; it prints one line.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstring>
#include "gemm.hpp"
using namespace tps;
__global__ void fill_bf16(unsigned short* p, size_t n, unsigned seed) {
  for (size_t i = blockIdx.x * size_t(256) + threadIdx.x; i < n; i += size_t(gridDim.x) * 256) {
    unsigned x = unsigned(i) * 2654435761u + seed;
    x ^= x >> 13; x *= 0x5bd1e995u; x ^= x >> 15;
    float f = (float((x & 0xffff)) / 65536.0f - 0.5f) * 0.1f;
    p[i] = (unsigned short)(__float_as_uint(f) >> 16);
  }
}
int main(int argc, char** argv) {
  const int layout = argc > 1 && !strcmp(argv[1], "fwd") ? kFwd : kDgrad;
  const int M = 16384, N = 8192, K = 7168;
  unsigned short *A, *B, *C;
  if (hipMalloc(&A, size_t(M) * K * 2) || hipMalloc(&B, size_t(N) * K * 2) || hipMalloc(&C, size_t(M) * N * 2)) return 1;
  hipLaunchKernelGGL(fill_bf16, dim3(1024), dim3(256), 0, 0, A, size_t(M) * K, 1u);
  hipLaunchKernelGGL(fill_bf16, dim3(1024), dim3(256), 0, 0, B, size_t(N) * K, 2u);
  GemmArgs g{};
  g.A = A; g.B = B; g.C = C; g.M = M; g.N = N; g.K = K;
  g.lda = K; g.ldb = layout == kFwd ? K : N; g.ldc = N;  // kFwd B[N][K]; kDgrad B[K][N]
  for (int r = 0; r < 12; ++r)
    if (launch_gemm(g, layout, kEpiBf16, 0, nullptr, nullptr, kTile256x256w4, true) != hipSuccess) return 2;
  if (hipDeviceSynchronize()) return 3;
  printf("ok %s\n", layout == kFwd ? "fwd" : "dgrad");
  return 0;
}
