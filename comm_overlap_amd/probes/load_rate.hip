// Load-path probe: 1 block (4 waves) per CU streams 64 KB per iteration into LDS, then waits and
// synchronizes, like one k block of the 256 x 256 GEMM tile. Paths: direct buffer_load ... lds
// (dwordx4) against buffer_load_dwordx4 into registers followed by ds_write_b128.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <algorithm>
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// region: bytes per block (power of two); each iteration reads 64 KB at offset (it * 64 KB) % region
template <int MODE>
__global__ __launch_bounds__(256, 1) void probe(const char* src, uint32_t total, uint32_t region, int iters,
                                                int* out) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src, total);
  const uint32_t base = blockIdx.x * region;
  int acc = 0;
  for (int it = 0; it < iters; ++it) {
    const uint32_t off = base + ((uint32_t(it) * 65536u) & (region - 1));
    char* stage = smem + (it & 1) * 65536;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t o = off + (wave * 16 + j) * 1024 + lane * 16;
      if constexpr (MODE == 0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + (wave * 16 + j) * 1024), 16, o, 0, 0, 16);
      } else {
        i32x4 v = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        *reinterpret_cast<i32x4*>(stage + (wave * 16 + j) * 1024 + lane * 16) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0) expcnt(0)
    __syncthreads();
    acc += *reinterpret_cast<const int*>(smem + ((it & 1) * 65536) + t * 4);
  }
  out[blockIdx.x * 256 + t] = acc;
}

int main() {
  const uint32_t total = 1u << 30;  // 1 GiB source
  char* src; int* out;
  if (hipMalloc(&src, total) || hipMalloc(&out, 1024 * 256 * sizeof(int))) { printf("alloc\n"); return 1; }
  if (hipMemset(src, 1, total)) return 1;
  hipEvent_t e0, e1; (void)hipEventCreate(&e0); (void)hipEventCreate(&e1);
  (void)hipFuncSetAttribute((const void*)probe<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
  (void)hipFuncSetAttribute((const void*)probe<1>, hipFuncAttributeMaxDynamicSharedMemorySize, 131072);
  struct C { const char* name; int mode; uint32_t region; };
  const C cs[] = {{"dma  past L2 (256 KB/CU)", 0, 1u << 18}, {"vgpr past L2 (256 KB/CU)", 1, 1u << 18},
                  {"dma  HBM stream (4 MB/CU)", 0, 1u << 22}, {"vgpr HBM stream (4 MB/CU)", 1, 1u << 22},
                  {"dma  L2-resident (64 KB/CU)", 0, 1u << 16}, {"vgpr L2-resident (64 KB/CU)", 1, 1u << 16}};
  for (int rep = 0; rep < 2; ++rep)
  for (const C& c : cs) {
    const int blocks = 256, iters = 2000;
    if (uint64_t(blocks) * c.region > total) { printf("too big\n"); return 1; }
    auto launch = [&]() {
      if (c.mode == 0) hipLaunchKernelGGL(probe<0>, dim3(blocks), dim3(256), 131072, 0, src, total, c.region, iters, out);
      else hipLaunchKernelGGL(probe<1>, dim3(blocks), dim3(256), 131072, 0, src, total, c.region, iters, out);
    };
    launch();
    if (hipDeviceSynchronize()) { printf("sync\n"); return 1; }
    std::vector<float> ts;
    for (int r = 0; r < 5; ++r) {
      (void)hipEventRecord(e0, 0); launch(); (void)hipEventRecord(e1, 0); (void)hipEventSynchronize(e1);
      float ms; (void)hipEventElapsedTime(&ms, e0, e1); ts.push_back(ms);
    }
    std::sort(ts.begin(), ts.end());
    const double bytes = double(blocks) * iters * 65536.0;
    const double per_cu_clk = 65536.0 * iters / (ts[2] * 1e-3 * 2.3e9);
    printf("%-32s %8.3f ms  %7.1f TB/s total  %5.1f B/clk/CU at 2.3 GHz\n", c.name, ts[2], bytes / (ts[2] * 1e-3) / 1e12,
           per_cu_clk);
  }
  return 0;
}
