// Read bandwidth of the memory hierarchy, for the rooflines of the kernels
// that live on cache reuse (attention over small cubes): every workgroup
// reads 4 MiB with 16-byte loads, eight in flight per thread, from a window
// of S bytes, wrapping, from a workgroup-dependent start; S = 2 MiB stays in each XCD's L2, 16 to
// 128 MiB stay in the memory-side cache (MALL), 2 GiB streams from HBM.
// Prints one JSON object (GB/s, median of three timed runs after one warm
// run). Built next to the library; run by the benchmark's --cache-bandwidth.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

// Every thread keeps kInFlight independent 16-byte loads in flight (a single
// load per thread would measure the latency of the level, not its
// bandwidth). Windows are powers of two, so the wrap is a mask.
constexpr int kInFlight = 8;

__global__ __launch_bounds__(256) void read_window(const f32x4* __restrict__ buf, size_t mask, size_t per_block,
                                                   float* __restrict__ out) {
  const size_t start = ((size_t)blockIdx.x * 4099u * 256u) & mask;
  f32x4 acc[kInFlight];
#pragma unroll
  for (int k = 0; k < kInFlight; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (size_t i = threadIdx.x; i < per_block; i += 256 * kInFlight) {
    f32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = buf[(start + i + (size_t)k * 256) & mask];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc[k] += v[k];
  }
  f32x4 t = acc[0];
#pragma unroll
  for (int k = 1; k < kInFlight; ++k) t += acc[k];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = t[0] + t[1] + t[2] + t[3];
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "cache_probe: %s: %s\n", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

}  // namespace

int main() {
  const size_t max_bytes = (size_t)2 << 30;
  const int blocks = 256 * 16;
  const size_t per_block = (size_t)1 << 18;   // float4 loads per workgroup (4 MiB)
  f32x4* buf = nullptr;
  float* out = nullptr;
  if (!ok(hipMalloc(&buf, max_bytes), "hipMalloc") || !ok(hipMemset(buf, 0, max_bytes), "hipMemset") ||
      !ok(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)), "hipMalloc"))
    return 1;
  hipEvent_t e0, e1;
  if (!ok(hipEventCreate(&e0), "event") || !ok(hipEventCreate(&e1), "event")) return 1;
  const size_t wins[] = {(size_t)2 << 20, (size_t)16 << 20, (size_t)64 << 20, (size_t)128 << 20, max_bytes};
  std::printf("{\"read_gbs\": {");
  bool first = true;
  for (size_t w : wins) {
    const size_t mask = w / 16 - 1;   // windows are powers of two
    std::vector<float> ms;
    for (int rep = 0; rep < 4; ++rep) {
      if (!ok(hipEventRecord(e0), "record")) return 1;
      hipLaunchKernelGGL(read_window, dim3(blocks), dim3(256), 0, 0, buf, mask, per_block, out);
      if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") ||
          !ok(hipEventSynchronize(e1), "sync"))
        return 1;
      float t = 0.f;
      if (!ok(hipEventElapsedTime(&t, e0, e1), "elapsed")) return 1;
      if (rep > 0) ms.push_back(t);
    }
    std::sort(ms.begin(), ms.end());
    const double bytes = (double)blocks * per_block * 16;
    std::printf("%s\"%zuMiB\": %.1f", first ? "" : ", ", w >> 20, bytes / ms[1] / 1e6);
    first = false;
  }
  std::printf("}, \"bytes_per_window\": %.0f}\n", (double)blocks * per_block * 16);
  (void)hipFree(buf);
  (void)hipFree(out);
  return 0;
}
