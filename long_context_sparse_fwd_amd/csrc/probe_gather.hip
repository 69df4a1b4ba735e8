// Gather-bandwidth probe for the selected-block branch.
//
// The selected branch of NSA (the sparse-selection passage of the pages'
// fine-grained branch) reads, for every query token, its chosen 64-token
// blocks of K and V. On i.i.d. inputs the choices are effectively random, so
// the kernel is a stream of random 16 KiB half-block reads (16 loads of 1 KiB
// per wave, as the prefill kernel issues them) over one KV group's tiles. This
// program measures what the chip delivers for exactly that pattern, as a
// function of the working set each XCD draws from (one KV group's K and V
// tiles at 64k tokens are 32 MiB; an XCD's L2 is 4 MiB; the Infinity Cache
// is 256 MiB).
//
// Launch shape as in the prefill kernel: one workgroup of 4 waves per CU
// (the LDS request keeps a second one out), workgroup i on XCD i % 8; XCD x
// draws from region x / 2 of the buffer, so two XCDs share a region like two
// XCDs share a KV group. U = half blocks in flight per wave.
//
// Usage: probe_gather [iters]   (prints one line per working set and U)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                       \
    }                                                                                     \
  } while (0)

namespace {

constexpr size_t kHalf = 16384;  // bytes of one half block (32 keys x 128 x bf16, K or V)
constexpr int kWaves = 4;

// a 32-bit integer mixer (the "lowbias32" constants of Chris Wellons' hash
// prospector); only used to spread the block choices
__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int U>
__global__ __launch_bounds__(256) void gather(const unsigned char* __restrict__ buf, size_t region, int iters,
                                              uint4* sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned char* base = buf + static_cast<size_t>((blockIdx.x & 7) >> 1) * region;
  const unsigned nhalf = static_cast<unsigned>(region / kHalf);
  const unsigned wid = blockIdx.x * kWaves + wave;
  uint4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; it += U) {
    uint4 r[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned j = mix(wid * 65537u + static_cast<unsigned>(it + u)) % nhalf;
      const unsigned char* p = base + static_cast<size_t>(j) * kHalf + 16 * lane;
#pragma unroll
      for (int f = 0; f < 16; ++f) r[u][f] = *reinterpret_cast<const uint4*>(p + 1024 * f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        acc.x ^= r[u][f].x;
        acc.y += r[u][f].y;
        acc.z ^= r[u][f].z;
        acc.w += r[u][f].w;
      }
  }
  // keeps the loads alive; the buffer is filled with a constant, so never taken
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[blockIdx.x] = acc;
}

template <int U>
void run(const unsigned char* buf, size_t region, int iters, int grid, uint4* sink) {
  // more than half of a CU's 160 KiB of LDS: one workgroup per CU
  const size_t lds = 96 * 1024;
  CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&gather<U>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int w = 0; w < 2; ++w) hipLaunchKernelGGL(gather<U>, dim3(grid), dim3(256), lds, 0, buf, region, iters, sink);
  CHECK(hipGetLastError());
  constexpr int kReps = 5;
  CHECK(hipEventRecord(e0));
  for (int rep = 0; rep < kReps; ++rep)
    hipLaunchKernelGGL(gather<U>, dim3(grid), dim3(256), lds, 0, buf, region, iters, sink);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  ms /= kReps;
  const double bytes = static_cast<double>(grid) * kWaves * iters * kHalf;
  std::printf("working set %6.1f MiB per XCD  U=%d  %8.3f ms  %6.2f TB/s delivered\n",
              region / 1048576.0, U, ms, bytes / (ms * 1e-3) / 1e12);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 256;
  if (iters <= 0 || iters % 4 != 0) {
    std::fprintf(stderr, "iters must be a positive multiple of 4\n");
    return 2;
  }
  int dev = 0, ncu = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  const int grid = ncu / 8 * 8;
  if (grid == 0) {
    std::fprintf(stderr, "unexpected CU count %d\n", ncu);
    return 2;
  }
  const size_t regions[] = {size_t{2} << 20, size_t{4} << 20, size_t{8} << 20,
                            size_t{16} << 20, size_t{32} << 20, size_t{64} << 20};
  const size_t max_region = size_t{64} << 20;
  // four regions (XCD x reads region x / 2); every read lies in
  // [region_index * region, region_index * region + region) with region <= max_region
  unsigned char* buf = nullptr;
  uint4* sink = nullptr;
  CHECK(hipMalloc(&buf, 4 * max_region));
  CHECK(hipMalloc(&sink, static_cast<size_t>(grid) * sizeof(uint4)));
  CHECK(hipMemset(buf, 1, 4 * max_region));
  std::printf("CUs %d, grid %d x 256 threads, %d half-block reads of 16 KiB per wave\n", ncu, grid, iters);
  for (size_t region : regions) {
    run<1>(buf, region, iters, grid, sink);
    run<2>(buf, region, iters, grid, sink);
    run<4>(buf, region, iters, grid, sink);
  }
  CHECK(hipDeviceSynchronize());
  CHECK(hipFree(buf));
  CHECK(hipFree(sink));
  return 0;
}
