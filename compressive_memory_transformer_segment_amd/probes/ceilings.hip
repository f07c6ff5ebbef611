// Practical ceilings of one MI355X (gfx950) for the rooflines the library reports against:
// the sustained rate of 32x32x16 bf16 matrix-core instructions (the instruction every
// matrix product of the library uses), the LDS read bandwidth per compute unit for the two
// operand reads the kernels use (ds_read_b128, ds_read_b64_tr_b16), and a device-to-device
// HBM copy.  Each figure comes from event-timed launches that fill every compute unit; the
// shader clock during a launch is derived from s_memtime against s_memrealtime (100 MHz).
//
// Build (build.py does this): hipcc --offload-arch=gfx950 -O3 ceilings.hip -o ceilings
// Run: ./ceilings   (prints one line per measurement)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

// Matrix-core rate: every wave runs `iters` rounds of NACC independent accumulation chains.
// zero_data selects all-zero operands (the matrix cores draw less power on zeros).
template <int NACC>
__global__ __launch_bounds__(512) void k_mfma(float* out, unsigned long long* clk, int iters, int zero_data) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[NACC];
  for (int a = 0; a < NACC; ++a)
    for (int r = 0; r < 16; ++r) acc[a][r] = 0.f;
  bf16x8 av, bv;
  for (int i = 0; i < 8; ++i) {
    const float x = zero_data ? 0.f : 0.01f * static_cast<float>(((lane * 37 + i * 11) % 61) - 30);
    const float y = zero_data ? 0.f : 0.01f * static_cast<float>(((lane * 13 + i * 29) % 53) - 26);
    av[i] = static_cast<__bf16>(x);
    bv[i] = static_cast<__bf16>(y);
  }
  const unsigned long long t0 = __builtin_readcyclecounter(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[a], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_readcyclecounter(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int a = 0; a < NACC; ++a)
    for (int r = 0; r < 16; ++r) s += acc[a][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// LDS read bandwidth: every wave reads `iters` x 16 operands of 1 KB (b128) or 512 B
// (transpose read) from a 64 KB region, consumed into an xor so that the reads stay live.
template <bool TR>
__global__ __launch_bounds__(1024) void k_lds(uint32_t* out, int iters) {
  __shared__ __align__(16) uint32_t lds[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = static_cast<uint32_t>(i) * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t acc = 0;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = (it * 16 + k + w * 3) & 63;
      if constexpr (TR) {
        const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(reinterpret_cast<uint16_t*>(lds) + ((row * 512 + lane * 4) & 32767)));
        acc ^= static_cast<uint32_t>(static_cast<uint16_t>(r[0])) ^ (static_cast<uint32_t>(static_cast<uint16_t>(r[3])) << 16);
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&lds[(row * 256 + lane * 4) & 16383]);
        acc ^= v[0] ^ v[3];
      }
    }
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

template <typename F>
float time_ms(F&& launch, int reps) {
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  launch();
  (void)hipDeviceSynchronize();
  (void)hipEventRecord(e0);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(e1);
  (void)hipEventSynchronize(e1);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms / reps;
}

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  std::printf("compute units: %d\n", cus);

  // matrix cores: one workgroup per compute unit, 4 or 8 waves (1 or 2 per SIMD)
  {
    float* out = nullptr;
    unsigned long long* clk = nullptr;
    CHECK(hipMalloc(&out, sizeof(float) * cus * 512));
    CHECK(hipMalloc(&clk, sizeof(unsigned long long) * 2 * cus));
    const int iters = 20000;
    for (int zero = 0; zero < 2; ++zero)
      for (int waves : {4, 8}) {
        const float ms = time_ms([&] { hipLaunchKernelGGL(k_mfma<4>, dim3(cus), dim3(64 * waves), 0, 0, out, clk, iters, zero); }, 3);
        std::vector<unsigned long long> c(2 * cus);
        CHECK(hipMemcpy(c.data(), clk, sizeof(unsigned long long) * 2 * cus, hipMemcpyDeviceToHost));
        double ghz = 0.0;
        for (int i = 0; i < cus; ++i) ghz += static_cast<double>(c[2 * i]) / (static_cast<double>(c[2 * i + 1]) * 10.0);
        ghz /= cus;
        const double flops = 2.0 * 32 * 32 * 16 * 4.0 * iters * waves * cus;
        std::printf("mfma 32x32x16 bf16, %s data, %d wave(s) per SIMD, 4 chains: %.0f TFLOP/s (shader clock %.2f GHz)\n",
                    zero ? "zero" : "nonzero", waves / 4, flops / (ms * 1e-3) / 1e12, ghz);
      }
    CHECK(hipFree(out));
    CHECK(hipFree(clk));
  }
  // LDS reads: one 16-wave workgroup per compute unit
  {
    uint32_t* out = nullptr;
    CHECK(hipMalloc(&out, sizeof(uint32_t) * cus));
    const int iters = 4000;
    const float ms128 = time_ms([&] { hipLaunchKernelGGL(k_lds<false>, dim3(cus), dim3(1024), 0, 0, out, iters); }, 3);
    const float mstr = time_ms([&] { hipLaunchKernelGGL(k_lds<true>, dim3(cus), dim3(1024), 0, 0, out, iters); }, 3);
    const double b128 = 1024.0 * 16 * iters * 16 * cus, btr = 512.0 * 16 * iters * 16 * cus;
    std::printf("lds ds_read_b128: %.1f TB/s total, %.0f GB/s per compute unit\n", b128 / (ms128 * 1e-3) / 1e12,
                b128 / cus / (ms128 * 1e-3) / 1e9);
    std::printf("lds ds_read_b64_tr_b16: %.1f TB/s total, %.0f GB/s per compute unit\n", btr / (mstr * 1e-3) / 1e12,
                btr / cus / (mstr * 1e-3) / 1e9);
    CHECK(hipFree(out));
  }
  // HBM: a 1 GiB device-to-device copy
  {
    const size_t bytes = size_t(1) << 30;
    u32x4 *a = nullptr, *b = nullptr;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMemset(a, 1, bytes));
    const size_t n = bytes / 16;
    const float ms = time_ms([&] { hipLaunchKernelGGL(k_copy, dim3(cus * 16), dim3(256), 0, 0, a, b, n); }, 5);
    std::printf("hbm copy 1 GiB: %.2f TB/s (read + write)\n", 2.0 * bytes / (ms * 1e-3) / 1e12);
    CHECK(hipFree(a));
    CHECK(hipFree(b));
  }
  return 0;
}
