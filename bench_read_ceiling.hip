// Streaming-read ceiling of the GPU's memory, the reference the decode
// kernel's HBM rate is read against: every 16-byte piece of a device buffer
// is read once per pass by a grid-stride loop and folded into one word per
// thread (the only write). It sweeps the grid size and the loads each thread
// keeps in flight, since more bytes in flight per CU is not always faster.
// Prints one JSON object per configuration and a final one with the best.
//
//     read_ceiling [GiB]      (default 16, about the K + V bytes of the
//                              packed decode batch)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ src, size_t n, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {  // all U loads of a pass are in bounds
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4_t v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

bool ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "read_ceiling: %s: %s\n", what, hipGetErrorString(e));
  return false;
}

template <int U>
double time_reads(const u32x4_t* buf, size_t n, uint32_t* out, int grid) {
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "hipEventCreate") || !ok(hipEventCreate(&b), "hipEventCreate")) return -1.0;
  for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(read_kernel<U>, dim3(grid), dim3(256), 0, 0, buf, n, out);
  if (!ok(hipDeviceSynchronize(), "warm-up")) return -1.0;
  const int reps = 10;
  (void)hipEventRecord(a, 0);
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(read_kernel<U>, dim3(grid), dim3(256), 0, 0, buf, n, out);
  (void)hipEventRecord(b, 0);
  if (!ok(hipEventSynchronize(b), "timed passes")) return -1.0;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return (double)n * 16.0 * reps / (ms * 1e-3) / 1e9;
}

}  // namespace

int main(int argc, char** argv) {
  const double gib = argc > 1 ? std::atof(argv[1]) : 16.0;
  if (!(gib > 0.0 && gib <= 64.0)) {
    std::fprintf(stderr, "read_ceiling: size must be in (0, 64] GiB\n");
    return 2;
  }
  const size_t n = (size_t)(gib * (double)(1ull << 30)) / 16;
  u32x4_t* buf = nullptr;
  uint32_t* out = nullptr;
  const int max_grid = 256 * 16;
  if (!ok(hipMalloc(&buf, n * 16), "hipMalloc") || !ok(hipMalloc(&out, (size_t)max_grid * 256 * 4), "hipMalloc"))
    return 1;
  if (!ok(hipMemset(buf, 1, n * 16), "hipMemset")) return 1;
  double best = 0.0;
  int best_grid = 0, best_u = 0;
  for (int grid : {256 * 4, 256 * 8, 256 * 16}) {
    for (int u : {1, 4}) {
      const double gbs = u == 1 ? time_reads<1>(buf, n, out, grid) : time_reads<4>(buf, n, out, grid);
      if (gbs < 0.0) return 1;
      std::printf("{\"grid\": %d, \"loads_in_flight_per_thread\": %d, \"GB/s\": %.1f}\n", grid, u, gbs);
      std::fflush(stdout);
      if (gbs > best) {
        best = gbs;
        best_grid = grid;
        best_u = u;
      }
    }
  }
  std::printf("{\"read_ceiling_GB/s\": %.1f, \"grid\": %d, \"loads_in_flight_per_thread\": %d, \"bytes\": %zu}\n", best,
              best_grid, best_u, n * 16);
  (void)hipFree(buf);
  (void)hipFree(out);
  return 0;
}
