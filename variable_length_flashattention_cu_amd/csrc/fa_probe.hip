// fa_probe.hip -- the matrix-core ceiling probe declared in include/fa_probe.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;   // 8 wavefronts: two per SIMD
constexpr int kChains = 8;      // independent accumulators per wavefront

struct WaveClock {
  long long cycles;  // shader clock ticks
  long long ticks;   // 100 MHz real-time ticks
};

// Each wavefront: `iters` x 8 independent MFMAs on register operands.  The
// operands come from the lane id so that the compiler cannot fold them; the
// accumulators are summed and written so that no MFMA is dead.
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float* out, WaveClock* clk) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, (uint32_t)lane, 0x3f80u});
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, (uint32_t)lane << 16, 0x3f803f80u, 0u});
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  out[blockIdx.x * kThreads + threadIdx.x] = s;
  if (lane == 0) {
    clk[wave].cycles = c1 - c0;
    clk[wave].ticks = r1 - r0;
  }
}

// 32-bit mixing function (the finaliser of MurmurHash3): operand bits only.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// Eight A and eight B fragments of pseudo-random bf16 values in +-[1, 2)
// (random sign and mantissa bits, so consecutive MFMAs switch their operand
// bits as attention data does); chain j multiplies A fragment j by B fragment
// (j + 1) % 8.
__global__ __launch_bounds__(kThreads) void mfma_peak_random_kernel(int iters, uint32_t seed, float* out,
                                                                    WaveClock* clk) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    u32x4 wa, wb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t ha = mix32(seed ^ mix32(gid * 64u + (uint32_t)(j * 8 + k)));
      const uint32_t hb = mix32(~seed ^ mix32(gid * 64u + (uint32_t)(j * 8 + k)));
      wa[k] = (ha & 0x807f807fu) | 0x3f803f80u;
      wb[k] = (hb & 0x807f807fu) | 0x3f803f80u;
    }
    a[j] = __builtin_bit_cast(bf16x8, wa);
    b[j] = __builtin_bit_cast(bf16x8, wb);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 1) % kChains], acc[j], 0, 0, 0);
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  out[blockIdx.x * kThreads + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) {
    clk[wave].cycles = c1 - c0;
    clk[wave].ticks = r1 - r0;
  }
}

// One warm-up launch, then one launch timed with HIP events; the clock is
// the mean over wavefronts of shader-clock ticks per real-time tick.
template <typename Launch>
int run_probe(int32_t iters, double* tflops, double* ghz, Launch&& launch) {
  if (!tflops || !ghz || iters < 1) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 8;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 8;
  const int grid = cus;  // one workgroup (8 wavefronts) per compute unit
  const int waves = grid * (kThreads / 64);
  float* out = nullptr;
  WaveClock* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 8;
  float ms = 0.f;
  if (hipMalloc((void**)&out, sizeof(float) * grid * kThreads) != hipSuccess) goto done;
  if (hipMalloc((void**)&clk, sizeof(WaveClock) * waves) != hipSuccess) goto done;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
  launch(grid, out, clk);  // warm-up
  if (hipGetLastError() != hipSuccess) goto done;
  if (hipEventRecord(e0, 0) != hipSuccess) goto done;
  launch(grid, out, clk);
  if (hipGetLastError() != hipSuccess) goto done;
  if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) goto done;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f) goto done;
  {
    WaveClock* h = new WaveClock[waves];
    if (hipMemcpy(h, clk, sizeof(WaveClock) * waves, hipMemcpyDeviceToHost) != hipSuccess) {
      delete[] h;
      goto done;
    }
    double sum = 0.0;
    int n = 0;
    for (int i = 0; i < waves; ++i)
      if (h[i].ticks > 0) {
        sum += (double)h[i].cycles / ((double)h[i].ticks * 10.0);  // ticks are 10 ns
        ++n;
      }
    delete[] h;
    const double flops = (double)waves * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
    *tflops = flops / ((double)ms * 1e-3) / 1e12;
    *ghz = n > 0 ? sum / n : 0.0;
    rc = 0;
  }
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (clk) (void)hipFree(clk);
  return rc;
}

}  // namespace

extern "C" int fa_probe_mfma_peak_random(int32_t iters, uint32_t seed, double* tflops, double* ghz) {
  return run_probe(iters, tflops, ghz, [&](int grid, float* out, WaveClock* clk) {
    hipLaunchKernelGGL(mfma_peak_random_kernel, dim3(grid), dim3(kThreads), 0, 0, iters, seed, out, clk);
  });
}

extern "C" int fa_probe_mfma_peak(int32_t iters, double* tflops, double* ghz) {
  return run_probe(iters, tflops, ghz, [&](int grid, float* out, WaveClock* clk) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(kThreads), 0, 0, iters, out, clk);
  });
}
