// Block compression of a K/V cache into a block-mean cache: entry j is the
// mean of tokens [64 j, 64 j + 64), non-overlapping (stride 64). The pages
// describe each key block being compressed into one representation (NSA
// factory write-up, chencunli.com, section "What dynamic sparsity actually
// sparsifies"); here the compression is the block mean, with the block size of
// the NSA how-to (qwbw.cn/news/106443), section 3. The summation order (token
// 0..63, fp32) and the single final rounding are the same as in the prefill
// re-layout kernel, so both phases see identical block means.
#include "nsa_device.h"
#include "nsa_internal.h"

namespace nsa {

template <class T>
__global__ __launch_bounds__(128) void k_compress(int D, const typename T::storage* k, int64_t ks0,
                                                  int64_t ks1, int64_t ks2,
                                                  const typename T::storage* v, int64_t vs0,
                                                  int64_t vs1, int64_t vs2, typename T::storage* kc,
                                                  int64_t kcs0, int64_t kcs1, int64_t kcs2,
                                                  typename T::storage* vc, int64_t vcs0,
                                                  int64_t vcs1, int64_t vcs2) {
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const typename T::storage* kp = k + b * ks0 + g * ks1 + static_cast<int64_t>(j) * 64 * ks2 + d;
    const typename T::storage* vp = v + b * vs0 + g * vs1 + static_cast<int64_t>(j) * 64 * vs2 + d;
    float sk = 0.f, sv = 0.f;
    for (int i = 0; i < 64; ++i) {
      sk += to_f32<T>(kp[i * ks2]);
      sv += to_f32<T>(vp[i * vs2]);
    }
    kc[b * kcs0 + g * kcs1 + static_cast<int64_t>(j) * kcs2 + d] = from_f32<T>(sk * (1.0f / 64.0f));
    vc[b * vcs0 + g * vcs1 + static_cast<int64_t>(j) * vcs2 + d] = from_f32<T>(sv * (1.0f / 64.0f));
  }
}

hipError_t launch_compress(int B, int G, int Nc, int D, bool bf16, const void* k, const int64_t* ks,
                           const void* v, const int64_t* vs, void* kc, const int64_t* kcs,
                           void* vc, const int64_t* vcs, hipStream_t st) {
  const dim3 grid(Nc, G, B);
  if (bf16) {
    hipLaunchKernelGGL(k_compress<BF16>, grid, dim3(128), 0, st, D, static_cast<const uint16_t*>(k),
                       ks[0], ks[1], ks[2], static_cast<const uint16_t*>(v), vs[0], vs[1], vs[2],
                       static_cast<uint16_t*>(kc), kcs[0], kcs[1], kcs[2],
                       static_cast<uint16_t*>(vc), vcs[0], vcs[1], vcs[2]);
  } else {
    hipLaunchKernelGGL(k_compress<F32>, grid, dim3(128), 0, st, D, static_cast<const float*>(k),
                       ks[0], ks[1], ks[2], static_cast<const float*>(v), vs[0], vs[1], vs[2],
                       static_cast<float*>(kc), kcs[0], kcs[1], kcs[2], static_cast<float*>(vc),
                       vcs[0], vcs[1], vcs[2]);
  }
  return hipGetLastError();
}

}  // namespace nsa
