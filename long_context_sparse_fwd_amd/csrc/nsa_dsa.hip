// Token-level sparse attention with a ReLU indexer (DeepSeek Sparse Attention,
// DSA) on gfx950: each query attends to the top-k tokens a lightweight
// multi-head indexer ranks highest, taking the core attention from O(L^2) to
// O(L*k) (DSA how-to, bjdmk.com.cn/news/5181035, sections 1, 3 and 4).
//
//  k_dsa_index  indexer scores I(t, s) = sum_j w[t, j] * ReLU(qi[t, j] . ki[s])
//               for s <= t. 16 query tokens per workgroup (8 waves x 2); the
//               64-token chunks of the indexer keys are staged once in LDS in
//               MFMA-fragment order and shared by the waves. The product
//               S = Qi . Ki^T puts the indexer heads on the MFMA rows, so a
//               lane holds 4 heads of one key: ReLU and the head weights in
//               registers, then the sum over the 4 lanes of a column with
//               the gfx950 lane swaps. Scores are written to a triangular
//               float32 buffer.
//  k_dsa_topk_fast   one workgroup per query row: a threshold from a
//               sample of the row, one read of the row that keeps the keys
//               above it in LDS, an exact radix select of the top-k among
//               them (ties to the lower token) and an ordered write of the
//               chosen tokens, ascending, padded with -1. A row whose sample
//               misses (too few or too many keys kept) is marked and left to
//  k_dsa_topk_exact  an exact radix select over the whole row (16 bits of
//               every order-preserving key cached in LDS).
//  k_dsa_attn   one workgroup per query token: the chosen tokens' K rows
//               (re-laid in MFMA-fragment order) and V rows (transposed) are
//               staged in LDS 32 at a time, double-buffered, and every wave
//               runs an online softmax for 16 query heads over them. Waves of
//               one KV head share its staging (one KV head for all query
//               heads is the absorbed-MLA form the page describes).
#include <algorithm>
#include <climits>
#include <type_traits>

#include "nsa_device.h"
#include "nsa_internal.h"

namespace nsa {
namespace {

template <class O>
__device__ __forceinline__ void store4(typename O::storage* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<BF16>(uint16_t* p, const f32x4& v) {
  uint2 w;
  w.x = pack_bf16x2(v.x, v.y);
  w.y = pack_bf16x2(v.z, v.w);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<F32>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

__device__ __forceinline__ int64_t score_row(const DsaArgs& a, int b, int t) {
  return static_cast<int64_t>(b) * a.L * (static_cast<int64_t>(a.L) + 1) / 2 +
         static_cast<int64_t>(t) * (t + 1) / 2;
}

// A 32-key piece of V^T in the A-operand order of the P.V product: the
// fragment of d-tile dt for lane l is 8 contiguous elements holding
// V[kappa(l/16, j)][16 dt + l%16] (kappa as for the 64-key V^T tiles: the keys
// whose probabilities lane l holds after the S^T product), in 16-byte slot
// dt*64 + 16 (l/16) + ((l%16) ^ (dt%8)): the XOR spreads a staging write of
// 16 lanes (one dim octet pair over eight d-tiles) over 16 bank groups.
__device__ __forceinline__ int vhalf_frag(int dt, int lane) {
  return (dt * 64 + 16 * (lane >> 4) + ((lane & 15) ^ (dt & 7))) * 8;
}
__device__ __forceinline__ int vhalf_off(int r, int d) {
  const int half = r >> 4, a = (r & 15) >> 2, i = r & 3;
  return vhalf_frag(d >> 4, (d & 15) + 16 * a) + 4 * half + i;
}

// K tiles of the bf16 kernels: the fragment-major layout of ktile_off with
// the 16-byte slots of each fragment XOR-swizzled, slot (r & 15) ^ m + 16 (m & 3)
// for key r and dim octet m = d / 8. A staging write of 16 lanes (one key,
// octets 0..15) then covers 16 distinct bank groups, and a fragment read of
// 16 lanes a permutation of 16 consecutive slots.
template <class T>
__device__ __forceinline__ int kchunk_off(int r, int d, int D) {
  if constexpr (sizeof(typename T::storage) == 2) {
    const int m = (d >> 3) & 15;
    return (((r >> 4) * (D >> 5) + (d >> 5)) * 64 + (((r & 15) ^ m) + 16 * (m & 3))) * 8;
  } else {
    return ktile_off(r, d, D);
  }
}
template <class T>
__device__ __forceinline__ int kfrag_off(int kt, int s, int lane, int D) {
  if constexpr (sizeof(typename T::storage) == 2) {
    const int m = (4 * s + (lane >> 4)) & 15;
    return ((kt * (D >> 5) + s) * 64 + (((lane & 15) ^ m) + 16 * (lane >> 4))) * 8;
  } else {
    return ktile_frag(kt, s, lane, D);
  }
}

// Staging position of 16-byte chunk e (8 elements of one key row) of a
// 32-key bf16 piece in the transposing order, D = 8 * NM with NM in {8, 16}:
// bits 0-3 of e (mlo) and 4-5 (i) come from the lane, the rest from the wave
// and slot; the chunk holds key 16h + 4a + i, dims 8m .. 8m + 7, with
// m = mlo % NM and (h, a) from the remaining bits. So the four lanes l, l^16,
// l^32, l^48 hold keys 4a + {0..3} of one dim octet and, in the chunk CH/2
// later, keys 16 + 4a + {0..3}: the eight keys of one V^T fragment.
template <int D>
__device__ __forceinline__ void stage_pos(int e, int& r, int& d) {
  constexpr int NM = D / 8;
  static_assert(NM == 8 || NM == 16, "head dims 64 and 128");
  const int mlo = e & 15, i = (e >> 4) & 3, rest = e >> 6;
  int a, h;
  if constexpr (NM == 16) {
    a = rest & 3;
    h = rest >> 2;
  } else {
    a = 2 * (rest & 1) + (mlo >> 3);
    h = rest >> 1;
  }
  r = 16 * h + 4 * a + i;
  d = 8 * (mlo % NM);
}

// v_permlane32_swap / v_permlane16_swap on a pair of registers: the upper
// 32 lanes of p trade with the lower 32 of q; odd 16-lane rows of p with even
// rows of q.
__device__ __forceinline__ void swap32(uint32_t& p, uint32_t& q) {
  const auto r = __builtin_amdgcn_permlane32_swap(p, q, false, false);
  p = r[0];
  q = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& p, uint32_t& q) {
  const auto r = __builtin_amdgcn_permlane16_swap(p, q, false, false);
  p = r[0];
  q = r[1];
}

// Four lanes l + 16 i (i = 0..3) each hold dwords D[0..3] of one key row
// (keys 4a + i, dims 8m .. 8m + 7); afterwards lane i holds in F[j] dword i of
// lane j's row, i.e. dims 8m + 2i and 8m + 2i + 1 of key 4a + j.
__device__ __forceinline__ void transpose4x4(const u32x4& x, uint32_t F[4]) {
  uint32_t p0 = x[0], p1 = x[1], q0 = x[2], q1 = x[3];
  swap32(p0, q0);  // p: rows of lanes with i < 2, q: of lanes with i >= 2; dwords 2 (i >> 1) + {0, 1}
  swap32(p1, q1);
  swap16(p0, p1);  // p0 from i = 0, p1 from i = 1, dword i of the source
  swap16(q0, q1);
  F[0] = p0;
  F[1] = p1;
  F[2] = q0;
  F[3] = q1;
}

// Unsigned key that orders like the float (larger float -> larger key).
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ k_dsa_index


template <class T, int DI>
__global__ __launch_bounds__(512) void k_dsa_index(DsaArgs a) {
  using S = typename T::storage;
  constexpr int KS = DI / 32, TILE = 64 * DI, NT = 64 * kIdxWaves;
  constexpr int EPC = 16 / static_cast<int>(sizeof(S));  // elements per 16-byte chunk
  constexpr int CH = TILE / EPC, PER = CH / NT;           // chunks of a tile, per thread
  static_assert(CH % NT == 0, "tile chunks must divide evenly");
  __shared__ __align__(16) S stage[2][TILE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = a.idx_tiles - 1 - static_cast<int>(blockIdx.x) / a.B;  // heaviest first
  const int b = static_cast<int>(blockIdx.x) % a.B;
  const int T0 = tile * kIdxTPW * kIdxWaves;
  if (T0 >= a.L) return;
  const int col = lane & 15, grp = lane >> 4;
  const int tw = T0 + kIdxTPW * wave;
  const int Tl = min(T0 + kIdxTPW * kIdxWaves - 1, a.L - 1);
  const S* QI = static_cast<const S*>(a.qi) + b * a.qis[0];
  const S* KI = static_cast<const S*>(a.ki) + b * a.kis[0];
  const S* W = static_cast<const S*>(a.w) + b * a.wis[0];

  // A operand: indexer head `col`, dims 32 s + 8 grp + j; the lane's C rows
  // are heads 4 grp + i, whose weights it keeps
  Frag<T> qf[kIdxTPW][KS];
  float wv[kIdxTPW][4];
  // reads at clamped (token, head) indices, all in flight together, zeroed where not valid
#pragma unroll
  for (int qt = 0; qt < kIdxTPW; ++qt) {
    const int t = tw + qt, tc = min(t, a.L - 1);
    const bool ok = t < a.L && col < a.Hi;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = frag_load_if<T>(
          QI + static_cast<int64_t>(tc) * a.qis[1] + min(col, a.Hi - 1) * a.qis[2] + 32 * s + 8 * grp, ok);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      const float x = to_f32<T>(W[static_cast<int64_t>(tc) * a.wis[1] + min(h, a.Hi - 1)]);
      wv[qt][i] = (t < a.L && h < a.Hi) ? x : 0.f;
    }
  }

  // 16-byte chunk e of chunk c: key row r, dims d .. d + EPC - 1 -> its place
  // in the fragment-major tile. Two register sets: chunk j travels in set
  // j & 1, issued two chunks before it is computed; keys past the sequence
  // read its last key instead (their scores are never stored).
  u32x4 reg[2][PER];
  auto issue = [&](int c, auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NT * i, r = (e * EPC) / DI, d = (e * EPC) % DI, key = min(64 * c + r, a.L - 1);
      reg[set][i] = *reinterpret_cast<const u32x4*>(KI + static_cast<int64_t>(key) * a.kis[1] + d);
    }
  };
  auto commit = [&](int buf, auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NT * i, r = (e * EPC) / DI, d = (e * EPC) % DI;
      *reinterpret_cast<u32x4*>(&stage[buf][kchunk_off<T>(r, d, DI)]) = reg[set][i];
    }
  };
  float* SC = a.scores;
  float* sink = a.scores + static_cast<int64_t>(a.B) * a.L * (static_cast<int64_t>(a.L) + 1) / 2;
  int64_t rows[kIdxTPW];
  // w * ReLU(x) is computed as (w / 2) * (x + |x|): the same product (x + |x|
  // is 2x or +0, and halving w is exact for normal w), in two instructions
  // where fmaxf needs three (it quiets NaN inputs first)
  float hw[kIdxTPW][4];
#pragma unroll
  for (int qt = 0; qt < kIdxTPW; ++qt) {
    rows[qt] = score_row(a, b, min(tw + qt, a.L - 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) hw[qt][i] = 0.5f * wv[qt][i];
  }
  auto compute = [&](int c) {
    const int buf = c & 1;
    // after the column sum every lane of a column holds the key's score; lane
    // (col, grp) keeps the one of 16-key tile kt = grp, so that one store per
    // token writes the chunk's 64 scores (key 64 c + lane)
    float mine[kIdxTPW] = {};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      Frag<T> kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = frag_load<T>(&stage[buf][kfrag_off<T>(kt, s, lane, DI)]);
#pragma unroll
      for (int qt = 0; qt < kIdxTPW; ++qt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(acc, qf[qt][s], kf[s]);
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(hw[qt][i], acc[i] + fabsf(acc[i]), v);
        // heads 4 grp .. 4 grp + 3 of the four lanes of this column
        v = col_sum4_fast(v);
        mine[qt] = grp == kt ? v : mine[qt];
      }
    }
    // lanes without a score to write (keys after the token) store to the
    // sink after the scores instead: no branch around the stores, so the
    // compiler's count of stores in flight is the same on every path
    const int key = 64 * c + lane;
#pragma unroll
    for (int qt = 0; qt < kIdxTPW; ++qt) {
      const int t = tw + qt;
      float* dst = (t < a.L && key <= t) ? SC + rows[qt] + key : sink + lane;
      *dst = mine[qt] + 0.f;   // + 0 turns -0 into +0
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  const int nch = (Tl >> 6) + 1;
  issue(0, Set0{});
  issue(min(1, nch - 1), Set1{});
  commit(0, Set0{});
  lds_barrier();
  // chunk c: issue c + 2 into the set chunk c came in (committed a step ago),
  // compute c, commit c + 1 (from `next_c`) into the buffer read at c - 1.
  // Every step issues and commits, chunks past the last one clamped to it,
  // and steps run in pairs (an odd count computes one chunk past the last,
  // whose keys follow every token, so nothing is stored): the loads in
  // flight are then the same on every path, and the compiler's waits cover
  // only the chunk being committed, not the one just issued.
  auto step = [&](int c, auto next_c) __attribute__((always_inline)) {
    constexpr int nxt = decltype(next_c)::value;
    issue(min(c + 2, nch - 1), std::integral_constant<int, 1 - nxt>{});
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the chunk's work
    compute(c);
    __builtin_amdgcn_sched_barrier(0);   // and the commit after it
    commit((c + 1) & 1, next_c);
    lds_barrier();
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, Set1{});
    step(c + 1, Set0{});
  }
}

// ------------------------------------------------------------------ k_dsa_topk

constexpr int kTopkThreads = 512, kTopkWaves = kTopkThreads / 64;
constexpr int kTopkCand = 1024;   // exact keys kept for the candidates sharing the boundary's top 16 bits

// Exclusive prefix sum of v over the workgroup (thread order) and its total.
// wsum: kTopkWaves words of LDS; synchronises once, and the caller must
// synchronise again before wsum is reused.
template <int NW = kTopkWaves>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total, int lane, int wave) {
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  lds_barrier();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return before + x - v;
}

// The bin holding the `need`-th largest element (1-based) of a histogram of
// nb bins (nb <= 8 * kTopkThreads, a multiple of 8 when above kTopkThreads),
// and that element's rank inside the bin, found by the whole workgroup:
// thread i sums the bins of slice kTopkThreads - 1 - i (thread 0 the highest
// bins), an exclusive scan gives the count above each slice, and the thread
// whose slice holds the element writes result[0..1]. The caller synchronises
// before reading result or reusing wsum.
template <int NTH = kTopkThreads>
__device__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* wsum, uint32_t* result, int tid,
                         int lane, int wave) {
  const int per = nb > NTH ? nb / NTH : 1;
  const int lo = (NTH - 1 - tid) * per, hi = min(nb, lo + per);
  uint32_t c[8];
  uint32_t sum = 0;
  if (per == 8) {
    const uint4 x = *reinterpret_cast<const uint4*>(hist + lo), y = *reinterpret_cast<const uint4*>(hist + lo + 4);
    c[0] = x.x, c[1] = x.y, c[2] = x.z, c[3] = x.w, c[4] = y.x, c[5] = y.y, c[6] = y.z, c[7] = y.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = lo + j < hi ? hist[lo + j] : 0u;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += c[j];
  uint32_t tot;
  uint32_t above = block_excl_scan<NTH / 64>(sum, wsum, &tot, lane, wave);
#pragma unroll
  for (int j = 7; j >= 0; --j) {
    if (lo + j < hi && above < need && need <= above + c[j]) {
      result[0] = static_cast<uint32_t>(lo + j);
      result[1] = need - above;
    }
    above += c[j];
  }
}

constexpr int kFastThreads = 256, kFastWaves = kFastThreads / 64;
constexpr int kFastCap = 3584;     // candidate keys a row may keep
constexpr int kFastSample = 4096;  // sampled scores: 16 evenly spaced runs of kFastThreads
constexpr int kTopkRedo = -2;      // first entry of a row the sampled pass leaves to the exact one
constexpr int kRedoRows = 256;     // rows whose markers one exact-pass workgroup checks
static_assert(kFastSample == 16 * kFastThreads, "one sampled score per thread and run");
static_assert(kDsaMaxTopK < kFastCap && kFastSample * 4 <= kFastCap * 8, "capacity above top_k; the sample fits the list");

// Top-k of one row of indexer scores by a sampled threshold (one workgroup
// per row; the chosen set is the exact one, as in k_dsa_topk_exact).
// 1. Rows longer than kFastCap: the orderable keys of 16 evenly spaced runs
//    of 256 scores; two 11-bit digits of a radix select give a threshold
//    theta (a 22-bit prefix) at or below the sample's r-th largest key, with
//    r chosen so that about (top_k + kFastCap) / 2 keys of the row are
//    expected at or above it. Shorter rows keep every key (theta = 0).
// 2. One read of the row: every key >= theta goes to an LDS list as a 64-bit
//    key (orderable score, complement of the token), each lane counting its
//    keys first so that a wave takes its places with one atomic.
// 3. If the list holds fewer than top_k keys, or more than kFastCap, the
//    sample missed: the row's first entry is set to kTopkRedo and the exact
//    pass redoes the row. Otherwise the top_k largest keys of the row are
//    the top_k largest of the list (all of them pass theta): the k-th is
//    found by radix digits of 11, 11 and 10 bits over the score (then over
//    the token complement, only when the k-th score is shared by candidates
//    not all chosen), the chosen tokens marked in a bitmap of the row and
//    written ascending by a workgroup scan of the bitmap's popcounts.
__global__ __launch_bounds__(kFastThreads) void k_dsa_topk_fast(DsaArgs a) {
  extern __shared__ __align__(16) unsigned char tf_lds[];
  uint64_t* cand = reinterpret_cast<uint64_t*>(tf_lds);                  // kFastCap keys; first the sample
  uint32_t* hist = reinterpret_cast<uint32_t*>(tf_lds + kFastCap * 8);  // 2048 bins; later the row's bitmap (L / 32 words)
  __shared__ uint32_t res[2];
  __shared__ uint32_t wsum[kFastWaves];
  __shared__ uint32_t ncand;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / a.L), t = static_cast<int>(row % a.L);
  const int n = t + 1, k = a.topk;
  int32_t* out = a.idx + row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kFastThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* S = a.scores + score_row(a, b, t);

  // one radix digit over `items` entries: dig(i) is the digit of entry i, or
  // -1 for an entry outside the known prefix; returns the bin of the
  // need-th largest, its rank inside the bin and the bin's count
  auto radix = [&](int items, int nbins, auto&& dig, uint32_t need, uint32_t& bin, uint32_t& rank,
                   uint32_t& cnt) __attribute__((always_inline)) {
    for (int i = tid; i < nbins; i += kFastThreads) hist[i] = 0u;
    lds_barrier();
    for (int i = tid; i < items; i += kFastThreads) {
      const int d = dig(i);
      if (d >= 0) atomicAdd(&hist[d], 1u);
    }
    lds_barrier();
    find_bin<kFastThreads>(hist, nbins, need, wsum, res, tid, lane, wave);
    lds_barrier();
    bin = res[0];
    rank = res[1];
    cnt = hist[bin];
    lds_barrier();   // before hist and res are written again
  };

  // the row as a scalar head up to 16-byte alignment, 16-byte loads in
  // rounds of UNR per thread, a scalar tail
  const int head = min(n, static_cast<int>((4 - ((reinterpret_cast<uintptr_t>(S) >> 2) & 3)) & 3));
  const int nv = (n - head) >> 2;   // whole float4s after the head
  const int tail0 = head + 4 * nv;
  const f32x4* S4 = reinterpret_cast<const f32x4*>(S + head);
  constexpr int UNR = 4;
  // one round, at clamped indices (entries past nv are masked by the caller)
  auto load_round = [&](int base, f32x4 (&v)[UNR]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < UNR; ++j) v[j] = S4[max(0, min(base + tid + kFastThreads * j, nv - 1))];
  };
  f32x4 va[UNR];

  // 1. the threshold
  uint32_t theta = 0u;
  if (n > kFastCap) {
    uint32_t* skey = reinterpret_cast<uint32_t*>(cand);
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = S[r * (n - kFastThreads) / 15 + tid];
    load_round(0, va);   // the row's first round stays in flight across the sample's digits
#pragma unroll
    for (int r = 0; r < 16; ++r) skey[r * kFastThreads + tid] = orderable(x[r]);
    const uint32_t aim = static_cast<uint32_t>(k + kFastCap) / 2;
    const uint32_t r = min(static_cast<uint32_t>(kFastSample),
                           (aim * kFastSample + static_cast<uint32_t>(n) - 1) / static_cast<uint32_t>(n));
    uint32_t d1, r1, c1, d2, r2, c2;
    radix(kFastSample, 2048, [&](int i) { return static_cast<int>(skey[i] >> 21); }, r, d1, r1, c1);
    radix(kFastSample, 2048, [&](int i) {
      const uint32_t u = skey[i];
      return (u >> 21) == d1 ? static_cast<int>((u >> 10) & 2047u) : -1;
    }, r1, d2, r2, c2);
    theta = (d1 << 21) | (d2 << 10);
  } else if (nv > 0) {
    load_round(0, va);
  }

  // 2. the candidates: one read of the row (a scalar head up to 16-byte
  // alignment, 16-byte loads, a scalar tail)
  if (tid == 0) ncand = 0u;
  lds_barrier();
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  // the lane's passing keys in order, with its place from the wave's prefix
  // of the per-lane counts and one atomic per wave
  auto append = [&](uint32_t cnt, auto&& emit) __attribute__((always_inline)) {
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) {   // counts up to 64
      const uint64_t bal = __ballot((cnt >> bit) & 1u);
      pre += static_cast<uint32_t>(__popcll(bal & below)) << bit;
      tot += static_cast<uint32_t>(__popcll(bal)) << bit;
    }
    if (tot == 0u) return;
    uint32_t base = 0u;
    if (lane == 0) base = atomicAdd(&ncand, tot);
    base = __shfl(base, 0, 64) + pre;
    emit(base);
  };
  auto key_of = [](uint32_t u, int i) -> uint64_t {
    return (static_cast<uint64_t>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
  };
  {
    // head and tail: at most 3 + 3 scores, by threads 0..5
    const int i = tid < 3 ? tid : tail0 + tid - 3;
    const bool ok = tid < 3 ? tid < head : (tid < 6 && i < n);
    const float xi = S[ok ? i : 0];
    const uint32_t u = ok ? orderable(xi) : 0u;
    const bool pass = ok && u >= theta;
    append(pass ? 1u : 0u, [&](uint32_t pos) {
      if (pass && pos < static_cast<uint32_t>(kFastCap)) cand[pos] = key_of(u, i);
    });
  }
  for (int base = 0; base < nv; base += kFastThreads * UNR) {
    // the next round in flight while this one is sorted out (unconditional:
    // the last round reloads its own tail, so every path has the same loads
    // outstanding and the wait below is for this round's only)
    f32x4 v[UNR];
#pragma unroll
    for (int j = 0; j < UNR; ++j) v[j] = va[j];
    load_round(base + kFastThreads * UNR, va);
    uint32_t u[UNR][4];
    uint64_t msk = 0u;
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      const bool in = base + tid + kFastThreads * j < nv;
      const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u[j][c] = orderable(e[c]);
        msk |= (in && u[j][c] >= theta) ? 1ull << (4 * j + c) : 0ull;
      }
    }
    append(static_cast<uint32_t>(__popcll(msk)), [&](uint32_t pos) {
#pragma unroll
      for (int j = 0; j < UNR; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((msk >> (4 * j + c)) & 1ull) {
            if (pos < static_cast<uint32_t>(kFastCap))
              cand[pos] = key_of(u[j][c], head + 4 * (base + tid + kFastThreads * j) + c);
            ++pos;
          }
    });
  }
  lds_barrier();
  const uint32_t nc = ncand;
  if (nc < static_cast<uint32_t>(k) || nc > static_cast<uint32_t>(kFastCap)) {
    if (tid == 0) out[0] = kTopkRedo;
    return;
  }

  // 3. the k-th largest candidate key, digit by digit
  const int nci = static_cast<int>(nc);
  uint64_t pre = 0;
  uint32_t need = static_cast<uint32_t>(k), cnt = nc;
  bool whole_score = false;   // every candidate with the k-th score is chosen
  {
    constexpr int kLo[6] = {53, 42, 32, 21, 10, 0}, kW[6] = {11, 11, 10, 11, 11, 10};
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      if (p == 3 && cnt == need) {
        whole_score = true;
        break;
      }
      const int lo = kLo[p], w = kW[p];
      uint32_t d, rk;
      radix(nci, 1 << w, [&](int i) {
        const uint64_t x = cand[i];
        return (p == 0 || (x >> (lo + w)) == pre) ? static_cast<int>((x >> lo) & ((1u << w) - 1u)) : -1;
      }, need, d, rk, cnt);
      pre = (pre << w) | d;
      need = rk;
    }
  }
  const uint64_t kth = whole_score ? pre << 32 : pre;

  // 4. the chosen tokens in a bitmap of the row (over the histogram), then
  // written ascending
  uint32_t* bits = hist;
  const int nwords = (n + 31) >> 5;
  for (int i = tid; i < nwords; i += kFastThreads) bits[i] = 0u;
  lds_barrier();
  for (int i = tid; i < nci; i += kFastThreads) {
    const uint64_t x = cand[i];
    if (x >= kth) {
      const uint32_t tok = 0xFFFFFFFFu - static_cast<uint32_t>(x);
      atomicOr(&bits[tok >> 5], 1u << (tok & 31));
    }
  }
  lds_barrier();
  const int per = (nwords + kFastThreads - 1) / kFastThreads;
  const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
  uint32_t mine = 0;
  for (int w = w0; w < w1; ++w) mine += static_cast<uint32_t>(__popc(bits[w]));
  uint32_t tot;
  uint32_t pos = block_excl_scan<kFastWaves>(mine, wsum, &tot, lane, wave);
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m != 0u) {
      const int bit = __ffs(m) - 1;
      m &= m - 1u;
      if (pos < static_cast<uint32_t>(k)) out[pos] = 32 * w + bit;   // exactly k are chosen; the test bounds the store
      ++pos;
    }
  }
}

// Exact top-k of one row of indexer scores, for the rows the sampled pass
// (k_dsa_topk_fast) left undone (first entry kTopkRedo): the chosen tokens
// are the k largest 64-bit keys (orderable score, complement of the token),
// so equal scores go to the lower token. The top 16 bits of every key are
// kept in LDS (the row is read from memory once, up to 65536 candidates); a
// 12-bit and a 4-bit digit find the top-16-bit value P of the k-th key; the
// candidates whose top 16 bits equal P are re-read, ranked by their exact
// keys and the chosen ones marked in a bitmap. With more than kTopkCand such
// candidates (heavy ties), the remaining 48 key bits are resolved by 8-bit
// digits instead. Then an ordered compaction writes the chosen tokens
// ascending. Each workgroup checks the markers of kRedoRows consecutive rows
// and runs the flagged ones in turn.
__global__ __launch_bounds__(kTopkThreads) void k_dsa_topk_exact(DsaArgs a) {
  extern __shared__ __align__(16) unsigned char tk_lds[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(tk_lds);                 // 4096 bins; later the bitmap
  uint64_t* cand = reinterpret_cast<uint64_t*>(tk_lds + 4096 * 4);     // kTopkCand exact keys
  uint16_t* c16 = reinterpret_cast<uint16_t*>(tk_lds + 4096 * 4 + kTopkCand * 8);  // top 16 bits of each key
  __shared__ uint32_t res[2];
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t ncand;
  __shared__ uint64_t kth_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int redo[kRedoRows];
  __shared__ int nredo;
  const int64_t rows = static_cast<int64_t>(a.B) * a.L, r0 = static_cast<int64_t>(blockIdx.x) * kRedoRows;
  if (tid == 0) nredo = 0;
  lds_barrier();
  if (tid < kRedoRows && r0 + tid < rows && a.idx[(r0 + tid) * a.topk] == kTopkRedo)
    redo[atomicAdd(&nredo, 1)] = tid;
  lds_barrier();
  const int nr = nredo;
  for (int f = 0; f < nr; ++f) {
    const int64_t row = r0 + redo[f];
    const int b = static_cast<int>(row / a.L), t = static_cast<int>(row % a.L);
    const int n = t + 1, k = a.topk;
    int32_t* out = a.idx + row * k;
    if (n <= k) {
      for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
      continue;
    }
    const float* S = a.scores + score_row(a, b, t);
    const int cap = a.topk_cache;   // c16 holds candidates [0, min(n, cap))
    auto top16 = [&](int i) -> uint32_t { return i < cap ? c16[i] : (orderable(S[i]) >> 16); };
    auto key64 = [&](int i) -> uint64_t {
      return (static_cast<uint64_t>(orderable(S[i])) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
    };

    // digit 1 (bits 31..20): one read of the row, sixteen loads in flight per thread
    for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0u;
    if (tid == 0) ncand = 0u;
    lds_barrier();
    auto take = [&](int i, float x) {
      const uint32_t u = orderable(x);
      if (i < cap) c16[i] = static_cast<uint16_t>(u >> 16);
      atomicAdd(&hist[u >> 20], 1u);
    };
    // the row starts at an arbitrary float: a scalar head up to 16-byte
    // alignment, then 16-byte loads (sixteen in flight per thread), a scalar tail
    const int head = min(n, static_cast<int>((4 - ((reinterpret_cast<uintptr_t>(S) >> 2) & 3)) & 3));
    if (tid < head) take(tid, S[tid]);
    const int nv = (n - head) >> 2;   // whole float4s after the head
    const f32x4* S4 = reinterpret_cast<const f32x4*>(S + head);
    constexpr int UNR = 4;
    for (int base = 0; base < nv; base += kTopkThreads * UNR) {
      f32x4 v[UNR];
  #pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int q4 = base + tid + kTopkThreads * j;
        v[j] = q4 < nv ? S4[q4] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
  #pragma unroll
      for (int j = 0; j < UNR; ++j) {
        const int q4 = base + tid + kTopkThreads * j;
        if (q4 < nv) {
          const int i = head + 4 * q4;
          take(i, v[j].x);
          take(i + 1, v[j].y);
          take(i + 2, v[j].z);
          take(i + 3, v[j].w);
        }
      }
    }
    for (int i = head + 4 * nv + tid; i < n; i += kTopkThreads) take(i, S[i]);
    lds_barrier();
    find_bin(hist, 4096, static_cast<uint32_t>(k), wsum, res, tid, lane, wave);
    lds_barrier();
    const uint32_t d1 = res[0], need1 = res[1];
    // passes over the cached top 16 bits, eight keys (one 16-byte word) at a time
    const int nq = min(n, cap) >> 3;   // whole words in the cache
    auto for_top16 = [&](auto&& f) {
      for (int q = tid; q < nq; q += kTopkThreads) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(c16 + 8 * q);
        const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
  #pragma unroll
        for (int j = 0; j < 8; ++j) f(8 * q + j, (ww[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      }
      for (int i = 8 * nq + tid; i < n; i += kTopkThreads) f(i, top16(i));
    };
    // digit 2 (bits 19..16) among the keys of bin d1
    if (tid < 16) hist[tid] = 0u;
    lds_barrier();
    for_top16([&](int, uint32_t c) {
      if ((c >> 4) == d1) atomicAdd(&hist[c & 15u], 1u);
    });
    lds_barrier();
    find_bin(hist, 16, need1, wsum, res, tid, lane, wave);
    lds_barrier();
    const uint32_t P = (d1 << 4) | res[0];
    uint32_t need = res[1];   // rank of the k-th key among the keys whose top 16 bits are P
    // the candidates sharing P: their exact keys
    for_top16([&](int i, uint32_t c) {
      if (c == P) {
        const uint32_t pos = atomicAdd(&ncand, 1u);
        if (pos < static_cast<uint32_t>(kTopkCand)) cand[pos] = key64(i);
      }
    });
    lds_barrier();
    const uint32_t nc = ncand;
    uint64_t kth;   // the k-th largest key of the row
    if (nc <= 256u) {
      // few candidates (the usual case): the k-th key is the one with exactly
      // need - 1 larger candidates (keys are distinct: they hold the token)
      for (int i = tid; i < static_cast<int>(nc); i += kTopkThreads) {
        const uint64_t x = cand[i];
        uint32_t above = 0;
        for (int j = 0; j < static_cast<int>(nc); ++j) above += cand[j] > x ? 1u : 0u;
        if (above == need - 1) kth_sh = x;
      }
      lds_barrier();
      kth = kth_sh;
    } else if (nc <= static_cast<uint32_t>(kTopkCand)) {
      // bitonic sort of the candidates, descending (zero keys pad to a power of two)
      int Pn = 1;
      while (Pn < static_cast<int>(nc)) Pn <<= 1;
      for (int i = static_cast<int>(nc) + tid; i < Pn; i += kTopkThreads) cand[i] = 0ull;
      lds_barrier();
      for (int size = 2; size <= Pn; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < Pn / 2; i += kTopkThreads) {
            const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
            const bool desc = (lo & size) == 0;
            const uint64_t x = cand[lo], y = cand[hi];
            if ((x < y) == desc) {
              cand[lo] = y;
              cand[hi] = x;
            }
          }
          lds_barrier();
        }
      kth = cand[need - 1];
    } else {
      // heavy ties: resolve the remaining 48 bits of the key by 8-bit digits
      uint64_t pre = P;   // the known high bits of the k-th key
      for (int shift = 40; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0u;
        lds_barrier();
        for (int i = tid; i < n; i += kTopkThreads)
          if (top16(i) == P) {
            const uint64_t kk = key64(i);
            if ((kk >> (shift + 8)) == pre) atomicAdd(&hist[(kk >> shift) & 0xFFu], 1u);
          }
        lds_barrier();
        find_bin(hist, 256, need, wsum, res, tid, lane, wave);
        lds_barrier();
        pre = (pre << 8) | res[0];
        need = res[1];
        lds_barrier();
      }
      kth = pre;
    }
    lds_barrier();
    // bitmap (over the histogram) of the chosen candidates sharing P
    uint32_t* bits = hist;
    const int nwords = (n + 31) >> 5;
    for (int i = tid; i < nwords; i += kTopkThreads) bits[i] = 0u;
    lds_barrier();
    if (nc <= static_cast<uint32_t>(kTopkCand)) {
      for (int i = tid; i < static_cast<int>(nc); i += kTopkThreads) {
        const uint64_t kk = cand[i];
        if (kk >= kth) {
          const uint32_t tok = 0xFFFFFFFFu - static_cast<uint32_t>(kk);
          atomicOr(&bits[tok >> 5], 1u << (tok & 31));
        }
      }
    } else {
      for (int i = tid; i < n; i += kTopkThreads)
        if (top16(i) == P && key64(i) >= kth) atomicOr(&bits[i >> 5], 1u << (i & 31));
    }
    lds_barrier();
    // ordered compaction: wave w takes the candidates [w * span, (w + 1) * span),
    // eight consecutive ones per lane and round; one workgroup scan of the wave
    // counts, then wave-level prefix sums
    const int span = ((n + 8 * kTopkThreads - 1) / (8 * kTopkThreads)) * 512;
    auto chosen8 = [&](int i0) -> uint32_t {   // bit j: candidate i0 + j is chosen
      uint32_t sel = 0;
      if (i0 < n) {
        uint16_t cc[8];
        if (i0 + 8 <= min(n, cap)) {
          const uint4 w4 = *reinterpret_cast<const uint4*>(c16 + i0);
          const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
  #pragma unroll
          for (int j = 0; j < 8; ++j) cc[j] = static_cast<uint16_t>(ww[j >> 1] >> (16 * (j & 1)));
        } else {
  #pragma unroll
          for (int j = 0; j < 8; ++j) cc[j] = i0 + j < n ? static_cast<uint16_t>(top16(i0 + j)) : 0;
        }
        const uint32_t mb = (bits[i0 >> 5] >> (i0 & 31)) & 0xFFu;
  #pragma unroll
        for (int j = 0; j < 8; ++j)
          if (i0 + j < n && (cc[j] > P || (cc[j] == P && ((mb >> j) & 1u)))) sel |= 1u << j;
      }
      return sel;
    };
    const int w0 = wave * span, w1 = min(n, w0 + span);
    uint32_t cnt = 0;
    for (int i0 = w0 + 8 * lane; i0 < w1; i0 += 512) cnt += static_cast<uint32_t>(__popc(chosen8(i0)));
    uint32_t tot;
    // the scan at lane 0 of a wave counts the chosen candidates of the lower waves
    uint32_t pos = __shfl(block_excl_scan(cnt, wsum, &tot, lane, wave), 0, 64);
    for (int r0 = w0; r0 < w1; r0 += 512) {
      const int i0 = r0 + 8 * lane;
      const uint32_t sel = i0 < w1 ? chosen8(i0) : 0u;
      const uint32_t c = static_cast<uint32_t>(__popc(sel));
      // inclusive prefix over the lanes of this round
      uint32_t x = c;
  #pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      uint32_t p = pos + x - c;
  #pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((sel >> j) & 1u) {
          if (p < static_cast<uint32_t>(k)) out[p] = i0 + j;   // exactly k are chosen; the test only bounds the store
          ++p;
        }
      pos += __shfl(x, 63, 64);
    }
    lds_barrier();   // the next row rewrites the LDS this one read
  }
}

// ------------------------------------------------------------------ k_dsa_attn

constexpr int kAttnBufs = 3;   // LDS buffers of 32 K rows + 32 V rows per KV head

template <class T, class O, int D, int WPG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(typename T::storage) == 2 ? 2 : 1))) void
k_dsa_attn(DsaArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int KS = D / 32, DT = D / 16, HALF = 32 * D;   // elements of a 32-key K piece or V^T piece
  constexpr int EPC = 16 / static_cast<int>(sizeof(S));
  constexpr int CH = HALF / EPC;                             // 16-byte chunks of a piece
  extern __shared__ __align__(16) unsigned char at_lds[];
  __shared__ int cnt_sh;
  __shared__ uint32_t wtot[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NTH = 64 * a.wg_waves;
  // workgroup (row, part): query token `row`, KV heads [part * gpw, part * gpw + gpw)
  const int64_t row = blockIdx.x / a.parts;
  const int part = static_cast<int>(blockIdx.x % a.parts);
  const int b = static_cast<int>(row / a.L), t = static_cast<int>(row % a.L);
  constexpr int wpg = WPG;                      // waves sharing one KV head (Hg / 16, or 1)
  const int gl = wave / wpg;                     // KV head of this wave within the workgroup
  const int gw = part * a.gpw + gl;              // ... and in the layer
  const int h0 = a.Hg >= 16 ? 16 * (part * a.wg_waves + wave) : gw * a.Hg;
  const int col = lane & 15, grp = lane >> 4;
  const bool colv = col < a.heads_per_wave;
  S* gbuf = reinterpret_cast<S*>(at_lds) + static_cast<size_t>(gl) * kAttnBufs * 2 * HALF;   // [buffers][K, V^T]
  int* list = reinterpret_cast<int*>(at_lds + static_cast<size_t>(a.gpw) * kAttnBufs * 2 * HALF * sizeof(S));
  int P = 1;
  while (P < a.topk) P <<= 1;
  int* tmp = list + P;

  // ---- this token's keys: ascending, distinct, each at or before t
  const int32_t* irow = a.idx + row * a.topk;
  if (tid == 0) cnt_sh = 0;
  lds_barrier();
  if (!a.inject) {
    // a computed row is ascending with -1 padding
    int c = 0;
    for (int i = tid; i < a.topk; i += NTH) {
      const int j = irow[i];
      list[i] = j;
      c += j >= 0 ? 1 : 0;
    }
    if (c) atomicAdd(&cnt_sh, c);
    lds_barrier();
  } else {
    // an injected row is a set of tokens: drop entries outside [0, t], sort, drop repeats
    for (int i = tid; i < P; i += NTH) {
      const int j = i < a.topk ? irow[i] : -1;
      tmp[i] = (j >= 0 && j <= t) ? j : INT_MAX;
    }
    lds_barrier();
    for (int size = 2; size <= P; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < P / 2; i += NTH) {
          const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
          const bool asc = (lo & size) == 0;
          const int x = tmp[lo], y = tmp[hi];
          if ((x > y) == asc) {
            tmp[lo] = y;
            tmp[hi] = x;
          }
        }
        lds_barrier();
      }
    // ordered compaction of the first occurrences
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int written = 0;
    for (int r0 = 0; r0 < P; r0 += NTH) {
      const int i = r0 + tid;
      const int x = i < P ? tmp[i] : INT_MAX;
      const bool keep = x != INT_MAX && (i == 0 || tmp[i - 1] != x);
      const uint64_t bal = __ballot(keep);
      if (lane == 0) wtot[wave] = static_cast<uint32_t>(__popcll(bal));
      lds_barrier();
      int before = __popcll(bal & below), tot = 0;
      for (int w = 0; w < a.wg_waves; ++w) {
        if (w < wave) before += static_cast<int>(wtot[w]);
        tot += static_cast<int>(wtot[w]);
      }
      if (keep) list[written + before] = x;
      written += tot;
      lds_barrier();
    }
    if (tid == 0) cnt_sh = written;
    lds_barrier();
  }
  const int cnt = cnt_sh;

  // ---- query fragments (B operand): head h0 + col, dims 32 s + 8 grp + j
  const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + static_cast<int64_t>(t) * a.qs[1] + (h0 + col) * a.qs[2] +
               8 * grp;
  Frag<T> qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = colv ? frag_load<T>(Q + 32 * s) : frag_zero<T>();

  // ---- staging: the waves of KV head gw copy its 32-key pieces
  const int gthreads = 64 * wpg, gt = (wave % wpg) * 64 + lane;
  const S* K = static_cast<const S*>(a.k) + b * a.ks[0] + gw * a.ks[2];
  const S* V = static_cast<const S*>(a.v) + b * a.vs[0] + gw * a.vs[2];
  constexpr int MAXPER = (CH + 64 * WPG - 1) / (64 * WPG);   // chunks per staging thread
  // bf16 with an even number of chunks per thread: V^T fragments are made in
  // registers (a 4 x 4 dword transpose over lanes l + 16 i, then half-word
  // packing) and stored with one 16-byte write each; otherwise V is written
  // element by element
  constexpr bool TR = EPC == 8 && CH % (128 * WPG) == 0;
  auto pos_of = [&](int e, int& r, int& d) {
    if constexpr (TR) {
      stage_pos<D>(e, r, d);
    } else {
      r = (e * EPC) / D;
      d = (e * EPC) % D;
    }
  };
  // two register sets: the rows of step j travel in set j & 1, issued two
  // steps before they are computed
  u32x4 rk[2][MAXPER], rv[2][MAXPER];
  // positions past the list read its last token's rows (masked out of the
  // softmax), so every load is unconditional and the loads in flight are the
  // same on every path (the compiler then waits only for the step committed)
  auto issue = [&](int step, auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int e = gt + gthreads * i;
      if (TR || e < CH) {
        int r, d;
        pos_of(e, r, d);
        const int64_t tok = list[min(32 * step + r, cnt - 1)];
        rk[set][i] = *reinterpret_cast<const u32x4*>(K + tok * a.ks[1] + d);
        rv[set][i] = *reinterpret_cast<const u32x4*>(V + tok * a.vs[1] + d);
      }
    }
  };
  auto commit = [&](int buf, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    S* kp = gbuf + buf * 2 * HALF;
    S* vp = kp + HALF;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int e = gt + gthreads * i;
      if (TR || e < CH) {
        int r, d;
        pos_of(e, r, d);
        *reinterpret_cast<u32x4*>(kp + kchunk_off<T>(r, d, D)) = rk[set][i];
        if constexpr (!TR) {
          const S* src = reinterpret_cast<const S*>(&rv[set][i]);
#pragma unroll
          for (int j = 0; j < EPC; ++j) vp[vhalf_off(r, d + j)] = src[j];
        }
      }
    }
    if constexpr (TR) {
      // slot i holds key 4a + i' (i' = lane / 16) and slot i + MAXPER / 2 key
      // 16 + 4a + i', dims 8m .. 8m + 7; lane i' ends with the fragments of
      // dims 8m + 2i' and 8m + 2i' + 1 (keys 4a + {0..3}, 16 + 4a + {0..3})
#pragma unroll
      for (int i = 0; i < MAXPER / 2; ++i) {
        const int e = gt + gthreads * i;
        int r, d;
        pos_of(e, r, d);
        uint32_t F0[4], F1[4];
        transpose4x4(rv[set][i], F0);
        transpose4x4(rv[set][i + MAXPER / 2], F1);
        const int ag = (r & 15) >> 2, dim = d + 2 * (lane >> 4);
        u32x4 lo, hi;   // fragments of dims `dim` (low halves) and `dim + 1` (high halves)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          lo[q] = (F0[2 * q] & 0xFFFFu) | (F0[2 * q + 1] << 16);
          hi[q] = (F0[2 * q] >> 16) | (F0[2 * q + 1] & 0xFFFF0000u);
          lo[2 + q] = (F1[2 * q] & 0xFFFFu) | (F1[2 * q + 1] << 16);
          hi[2 + q] = (F1[2 * q] >> 16) | (F1[2 * q + 1] & 0xFFFF0000u);
        }
        *reinterpret_cast<u32x4*>(vp + vhalf_frag(dim >> 4, (dim & 15) + 16 * ag)) = lo;
        *reinterpret_cast<u32x4*>(vp + vhalf_frag(dim >> 4, ((dim + 1) & 15) + 16 * ag)) = hi;
      }
    }
  };

  const float sl2 = a.scale_log2;
  float m = kNegBig, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsteps = (cnt + 31) >> 5;
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  if (nsteps > 0) {
    issue(0, Set0{});
    commit(0, Set0{});
    issue(min(1, nsteps - 1), Set1{});
    issue(min(2, nsteps - 1), Set0{});
    lds_barrier();
  }
  // one step; `next_c` is the register set of step + 1 (a constant: the loop runs steps in pairs)
  auto run_step = [&](int step, auto next_c) __attribute__((always_inline)) {
    const int buf = step % kAttnBufs;
    const S* kp = gbuf + buf * 2 * HALF;
    const S* vp = kp + HALF;
    f32x4 st[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      st[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) mma(st[h2], frag_load<T>(kp + kfrag_off<T>(h2, s, lane, D)), qf[s]);
    }
    Frag<T> vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vp + vhalf_frag(dt, lane));
    // positions past the list are masked out of the softmax (a step past
    // the last one is masked entirely)
    if (32 * step + 31 < cnt)
      online_step<T, DT, false>(st, 32 * step, 0, 0, grp, sl2, m, l, acc, vf);
    else
      online_step<T, DT, true>(st, 32 * step, 0, cnt - 1, grp, sl2, m, l, acc, vf);
    // step + 1's rows into the buffer last read at step - 2; then step + 3's
    // loads (clamped to the last step, as every step commits and issues)
    __builtin_amdgcn_sched_barrier(0);
    commit((step + 1) % kAttnBufs, next_c);
    issue(min(step + 3, nsteps - 1), next_c);
    lds_barrier();
  };
  // steps in pairs; with an odd count the last pair's second step is masked
  for (int step = 0; step < nsteps; step += 2) {
    run_step(step, Set1{});
    run_step(step + 1, Set0{});
  }

  const float lt = col_sum4(l);
  if (colv) {
    const float f = lt > 0.f ? 1.0f / lt : 0.f;
    SO* o = static_cast<SO*>(a.out) + b * a.os[0] + static_cast<int64_t>(t) * a.os[1] + (h0 + col) * a.os[2] + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) store4<O>(o + 16 * dt, acc[dt] * f);
  }
}

hipError_t record(hipEvent_t* ev, int i, hipStream_t st) {
  return ev != nullptr ? hipEventRecord(ev[i], st) : hipSuccess;
}

hipError_t launch_one(const void* fn, dim3 grid, dim3 block, size_t lds, hipStream_t st, const DsaArgs& a) {
  void* args[] = {const_cast<DsaArgs*>(&a)};
  return hipLaunchKernel(fn, grid, block, args, lds, st);
}

template <class T, class O, int D, int DI>
hipError_t launch_dsa_t(const DsaArgs& a, hipStream_t st, hipEvent_t* ev) {
  constexpr bool kBf16 = sizeof(typename T::storage) == 2;
  const int wpg = a.Hg >= 16 ? a.Hg / 16 : 1;
  const void* attn = wpg == 1   ? reinterpret_cast<const void*>(&k_dsa_attn<T, O, D, 1>)
                     : wpg == 2 ? reinterpret_cast<const void*>(&k_dsa_attn<T, O, D, 2>)
                     : wpg == 3 ? reinterpret_cast<const void*>(&k_dsa_attn<T, O, D, 3>)
                                : reinterpret_cast<const void*>(&k_dsa_attn<T, O, D, 4>);
  const void* topk = reinterpret_cast<const void*>(&k_dsa_topk_exact);
  const void* topk_fast = reinterpret_cast<const void*>(&k_dsa_topk_fast);
  const size_t attn_lds = dsa_attn_lds_bytes(a.gpw, D, kBf16, a.topk);
  const size_t topk_lds = dsa_topk_lds_bytes(a.topk_cache);
  // the candidate list, then the histogram or the row's bitmap
  const size_t fast_lds = kFastCap * sizeof(uint64_t) + std::max(2048, (a.L + 31) / 32) * sizeof(uint32_t);
  hipError_t e;
  if ((e = hipFuncSetAttribute(attn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(attn_lds))) !=
          hipSuccess ||
      (e = hipFuncSetAttribute(topk, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(topk_lds))) !=
          hipSuccess ||
      (e = hipFuncSetAttribute(topk_fast, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(fast_lds))) !=
          hipSuccess)
    return e;
  const unsigned rows = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.L);
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  if (!a.inject &&
      (e = launch_one(reinterpret_cast<const void*>(&k_dsa_index<T, DI>), dim3(a.B * a.idx_tiles), dim3(512), 0,
                      st, a)) != hipSuccess)
    return e;
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  // the sampled pass over every row, then the exact pass over the rows it left
  if (!a.inject && ((e = launch_one(topk_fast, dim3(rows), dim3(kFastThreads), fast_lds, st, a)) != hipSuccess ||
                    (e = launch_one(topk, dim3((rows + kRedoRows - 1) / kRedoRows), dim3(kTopkThreads), topk_lds,
                                    st, a)) != hipSuccess))
    return e;
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
  if ((e = launch_one(attn, dim3(rows * a.parts), dim3(64 * a.wg_waves), attn_lds, st, a)) != hipSuccess) return e;
  if ((e = record(ev, 3, st)) != hipSuccess) return e;
  return hipGetLastError();
}

template <class T, class O>
hipError_t launch_dsa_o(const DsaArgs& a, hipStream_t st, hipEvent_t* ev) {
  if (a.D == 64) return a.Di == 64 ? launch_dsa_t<T, O, 64, 64>(a, st, ev) : launch_dsa_t<T, O, 64, 128>(a, st, ev);
  return a.Di == 64 ? launch_dsa_t<T, O, 128, 64>(a, st, ev) : launch_dsa_t<T, O, 128, 128>(a, st, ev);
}

}  // namespace

size_t dsa_topk_lds_bytes(int cache) {
  return 4096 * sizeof(uint32_t) + kTopkCand * sizeof(uint64_t) + static_cast<size_t>(cache) * sizeof(uint16_t);
}

size_t dsa_attn_lds_bytes(int groups_per_wg, int D, bool bf16, int k) {
  int P = 1;
  while (P < k) P <<= 1;
  return static_cast<size_t>(groups_per_wg) * kAttnBufs * 2 * 32 * D * (bf16 ? 2 : 4) +
         2 * static_cast<size_t>(P) * sizeof(int);
}

hipError_t launch_dsa(const DsaArgs& a, bool in_bf16, bool out_bf16, hipStream_t st, hipEvent_t* ev) {
  if (in_bf16) return out_bf16 ? launch_dsa_o<BF16, BF16>(a, st, ev) : launch_dsa_o<BF16, F32>(a, st, ev);
  return launch_dsa_o<F32, F32>(a, st, ev);
}

}  // namespace nsa
