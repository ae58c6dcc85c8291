// Dense bf16 MFMA throughput this GPU sustains, with random and with constant
// operands: the practical ceiling of v_mfma_f32_16x16x32_bf16 (the attention
// kernel's instruction) under the board's clock and power management, which
// depends on the data's switching activity.  Every wave runs eight independent
// accumulator chains; operands cycle through eight register sets per lane.
// Prints one JSON line.  A measurement utility, not part of the library.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CK(x)                                                                \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                              \
    }                                                                        \
  } while (0)

constexpr int kSlots = 4096;  // operand slots; 16 bf16x8 each

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_stream(const bf16x8* __restrict__ src, float* out, long long* clk,
                                                   int iters) {
  const int slot = (blockIdx.x * 256 + threadIdx.x) & (kSlots - 1);
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[slot * 16 + i];
    b[i] = src[slot * 16 + 8 + i];
  }
  if (!RANDOM) {
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      a[i] = a[0];
      b[i] = b[0];
    }
  }
  f32x4 c[8] = {};
  const long long t0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(u + i) & 7], b[(u + 3 * i) & 7], c[i], 0, 0, 0);
  }
  const long long t1 = clock64(), w1 = wall_clock64();
  float s = 0.0f;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) s += c[i][j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 2] = t1 - t0;
    clk[blockIdx.x * 2 + 1] = w1 - w0;
  }
}

int main() {
  const int blocks = 2048, iters = 1024;
  const size_t n = (size_t)kSlots * 16;
  // random bf16 of magnitude ~[1/16, 4): random sign, exponent and mantissa
  std::vector<uint16_t> h(n * 8);
  uint64_t st = 0x9E3779B97F4A7C15ull;
  for (auto& v : h) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    const uint32_t r = (uint32_t)(st >> 33);
    v = (uint16_t)(((r & 1u) << 15) | ((123u + (r >> 1) % 7u) << 7) | ((r >> 4) & 0x7Fu));
  }
  bf16x8* d;
  float* o;
  long long* c;
  CK(hipMalloc(&d, n * sizeof(bf16x8)));
  CK(hipMalloc(&o, (size_t)blocks * 256 * sizeof(float)));
  CK(hipMalloc(&c, (size_t)blocks * 2 * sizeof(long long)));
  CK(hipMemcpy(d, h.data(), n * sizeof(bf16x8), hipMemcpyHostToDevice));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  double tf[2], ghz[2];
  for (int mode = 0; mode < 2; ++mode) {
    auto launch = [&] {
      if (mode == 0)
        hipLaunchKernelGGL(mfma_stream<true>, dim3(blocks), dim3(256), 0, 0, d, o, c, iters);
      else
        hipLaunchKernelGGL(mfma_stream<false>, dim3(blocks), dim3(256), 0, 0, d, o, c, iters);
    };
    for (int r = 0; r < 200; ++r) launch();  // ~1 s: the clock governor settles
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(e0));
    for (int r = 0; r < 50; ++r) launch();
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms;
    CK(hipEventElapsedTime(&ms, e0, e1));
    ms /= 50;
    long long hc[2];
    CK(hipMemcpy(hc, c, sizeof hc, hipMemcpyDeviceToHost));
    ghz[mode] = (double)hc[0] / (double)hc[1] * 0.1;  // wall_clock64 ticks at 100 MHz
    const double mfmas = (double)blocks * 4 * iters * 8 * 8;
    tf[mode] = mfmas * 16384.0 / (ms * 1e-3) / 1e12;
  }
  printf("{\"instruction\": \"v_mfma_f32_16x16x32_bf16\", \"random_tflops\": %.1f, \"random_clock_ghz\": %.3f, "
         "\"constant_tflops\": %.1f, \"constant_clock_ghz\": %.3f}\n",
         tf[0], ghz[0], tf[1], ghz[1]);
  return 0;
}
