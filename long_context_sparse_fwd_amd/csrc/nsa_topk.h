// Wave-level block selection: the query's own block plus the n-1 best-scoring
// earlier blocks, ties to the lower block index, written ascending and padded
// with -1. The score -> top-k -> gather dataflow follows the selector of the
// NSA factory write-up (chencunli.com, "DeepSeek NSA on the Siemens 840D
// manual"), section "What dynamic sparsity actually sparsifies"; the own-block
// rule and the tie rule are the readings stated in nsa.h.
//
// Method (exact, no approximation):
//  1. keys: score bits (scores are >= 0, so the unsigned bit pattern orders
//     like the float) with the top bit set to mark a real candidate, and, for
//     ordering, the 64-bit key (bits << 32) | (~j) which breaks ties to the
//     lower j;
//  2. theta = the (n-1)-th largest of the 64 per-lane maxima (bitonic sort
//     across lanes). At least n-1 candidates are >= theta, so every member of
//     the answer is >= theta;
//  3. the candidates >= theta (typically ~20) are compacted into LDS in
//     ascending block order. Up to 64 of them sit one per lane and each is
//     ranked by counting the larger keys; those of rank < n-1 are the
//     answer, already ascending, and the own block (the largest index) goes
//     last. With 65..kSurvCap survivors the ranks are counted the same way
//     from LDS; with more (heavy ties), n-1 rounds of wave-wide argmax over
//     all candidates are used instead; in both cases
//  4. the n chosen indices are sorted ascending across the lanes.
// The cross-lane sorts are bitonic networks whose exchanges inside 16-lane
// rows are DPP moves; only the 16- and 32-lane distances go through the LDS
// crossbar.
#pragma once

#include "nsa_device.h"
#include "nsa_internal.h"

namespace nsa {

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// The value of lane (lane ^ m), m a power of two below 64 (a constant after
// unrolling): DPP inside 16-lane rows (xor 4 as a half-row mirror followed by
// a reversed quad permutation), ds_swizzle across the rows of a 32-lane half,
// ds_bpermute across halves.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int m) {
  switch (m) {
    case 1: return dpp_u<0xB1>(v);                // quad_perm [1,0,3,2]
    case 2: return dpp_u<0x4E>(v);                // quad_perm [2,3,0,1]
    case 4: return dpp_u<0x1B>(dpp_u<0x141>(v));  // row_half_mirror, quad_perm [3,2,1,0]
    case 8: return dpp_u<0x128>(v);               // row_ror:8
    case 16: return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F));
    default: return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 32, 64));
  }
}
__device__ __forceinline__ uint64_t lane_xor(uint64_t v, int m) {
  const uint32_t lo = lane_xor(static_cast<uint32_t>(v), m);
  const uint32_t hi = lane_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// base + the number of set bits of m in the lanes below this one
__device__ __forceinline__ int mbcnt(uint64_t m, int base) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), static_cast<uint32_t>(base))));
}

// Bitonic sort of one value per lane across the wave: descending (lane 0
// holds the largest) or ascending.
template <bool DESC, class K>
__device__ __forceinline__ K wave_sort(K v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      const K o = lane_xor(v, jj);
      const bool first = ((lane & jj) == 0) == ((lane & k) == 0);
      v = (first == DESC) ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// sc: scores of blocks [0, own) in LDS (read by all lanes). out: n entries.
// surv: kSurvCap u64 of LDS scratch; selb: 64 ints of LDS scratch.
// Must be called by a whole wave with uniform arguments.
__device__ inline void topk_wave(const float* sc, int own, int n, int32_t* out, uint64_t* surv,
                                 int* selb, int lane) {
  const int n1 = n - 1;
  if (own <= n1) {
    if (lane < n) out[lane] = lane <= own ? lane : -1;
    return;
  }
  if (n1 == 0) {
    if (lane == 0) out[0] = own;
    return;
  }
  const int R = (own + 63) >> 6;
  // Keys of blocks lane + 64 (r0 + i), i < 8; the reads are unconditional
  // (indices clamped to own - 1) and independent, so they issue together.
  auto keys8 = [&](int r0, uint32_t (&k)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = lane + 64 * (r0 + i);
      const uint32_t bits = __float_as_uint(sc[min(j, own - 1)]);
      k[i] = j < own ? (bits | 0x80000000u) : 0u;
    }
  };
  uint32_t lmax = 0;
  for (int r0 = 0; r0 < R; r0 += 8) {
    uint32_t k[8];
    keys8(r0, k);
#pragma unroll
    for (int i = 0; i < 8; ++i) lmax = max(lmax, k[i]);
  }
  // theta: the (n-1)-th largest lane maximum
  const uint32_t theta = __builtin_amdgcn_readlane(wave_sort<true>(lmax, lane), n1 - 1);

  // the candidates >= theta, compacted into surv in ascending block order:
  // the eight rows' ballots first, then each survivor's place from v_mbcnt
  // and its store (the rows no longer wait on each other)
  int cnt = 0;
  for (int r0 = 0; r0 < R; r0 += 8) {
    uint32_t k[8];
    keys8(r0, k);
    bool f[8];
    uint64_t bal[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f[i] = k[i] >= theta && k[i] != 0u;
      bal[i] = __ballot(f[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pos = mbcnt(bal[i], cnt);  // cnt + survivors in lower lanes
      if (f[i] && pos < kSurvCap)
        surv[pos] = (static_cast<uint64_t>(k[i]) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - (lane + 64 * (r0 + i)));
      cnt += __popcll(bal[i]);
    }
  }
  wave_lds_sync();
  if (cnt <= 64) {
    // one survivor per lane; its rank = the number of larger keys (keys are
    // distinct). The n-1 of rank < n-1, taken in surv order, are already
    // ascending; the own block, larger than all of them, comes last.
    const uint64_t mine = lane < cnt ? surv[lane] : uint64_t{0};
    int rank = 0;
#pragma unroll 4
    for (int k = 0; k < cnt; ++k) rank += surv[k] > mine ? 1 : 0;
    const bool s = lane < cnt && rank < n1;
    const int pos = mbcnt(__ballot(s), 0);
    if (s) out[pos] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(mine));
    if (lane == 0) out[n1] = own;
    wave_lds_sync();
    return;
  }
  uint32_t jsel;  // this lane's chosen block (lanes < n), 0xFFFFFFFF elsewhere
  {
    if (cnt <= kSurvCap) {
      for (int i = lane; i < cnt; i += 64) {
        const uint64_t mine = surv[i];
        int rank = 0;
        for (int k = 0; k < cnt; ++k) rank += surv[k] > mine ? 1 : 0;
        if (rank < n1) selb[rank] = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(mine));
      }
    } else {
      uint64_t prev = ~0ull;
      for (int rr = 0; rr < n1; ++rr) {
        uint64_t best = 0;
        for (int j = lane; j < own; j += 64) {
          const uint64_t k64 =
              (static_cast<uint64_t>(__float_as_uint(sc[j]) | 0x80000000u) << 32) |
              static_cast<uint32_t>(0xFFFFFFFFu - j);
          if (k64 < prev && k64 > best) best = k64;
        }
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) {
          const uint64_t o = shfl_xor_u64(best, m);
          best = o > best ? o : best;
        }
        prev = best;
        if (lane == 0) selb[rr] = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
      }
    }
    wave_lds_sync();
    jsel = lane < n1 ? static_cast<uint32_t>(selb[lane]) : 0xFFFFFFFFu;
  }
  if (lane == n1) jsel = static_cast<uint32_t>(own);
  // the n chosen blocks in ascending order (the 0xFFFFFFFF fillers sort last)
  jsel = wave_sort<false>(jsel, lane);
  if (lane < n) out[lane] = static_cast<int32_t>(jsel);
  wave_lds_sync();
}

}  // namespace nsa
