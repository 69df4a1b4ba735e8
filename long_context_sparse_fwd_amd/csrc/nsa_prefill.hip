// NSA prefill on gfx950: three kernels per call.
//
//  k_prep     block compression + re-layout. One workgroup per 64-token block
//             (b, g, j): the block's K and V are staged in LDS, written back as
//             a fragment-major K tile and a permuted V^T tile, and, for
//             complete blocks, their fp32 means (the compressed keys/values)
//             are written into the compressed tiles. Compression by block
//             means, stride 64: compressed block representations, NSA factory
//             write-up (chencunli.com), section "What dynamic sparsity
//             actually sparsifies"; block size from the NSA how-to
//             (qwbw.cn/news/106443), section 3.
//  k_cmpwin   sliding-window branch + compressed branch + block scores +
//             top-k selection for 16 consecutive tokens of one KV group (8
//             waves, two per SIMD, each owning 2 tokens x 16 query heads).
//             Every 64-key tile the workgroup needs (window K/V blocks,
//             block-mean tiles, and at 8 waves the low parts of the K means)
//             is staged once in LDS, double-buffered, and shared by the 8
//             waves. The window output is normalised and gated first; the
//             compressed branch then adds gate_cmp * P . Vc into the same
//             accumulators (pass 1: log-sum-exp; pass 2: probabilities,
//             output, and block scores = probabilities summed over the
//             group's heads by a DPP reduce-scatter, kept in LDS). Each phase
//             runs its unmasked tiles and its masked edge tiles as separate
//             straight-line loops. The wave then selects each token's blocks.
//             Writes gate_win * O_win + gate_cmp * O_cmp into out and the
//             selection into idx. Workgroups run heaviest first.
//  k_sel      selected-block branch: a wave walks each of its tokens' chosen
//             blocks (32-key halves, the next one prefetched into registers
//             while the current one is computed), straight from the K/V tiles
//             in MFMA-fragment order; out += gate_slc * O_slc. One workgroup
//             per CU and work grouped by KV group per XCD: the random block
//             gathers are bound by L2-miss bandwidth, which fewer concurrent
//             waves per XCD use better.
#include <type_traits>

#include "nsa_device.h"
#include "nsa_internal.h"
#include "nsa_topk.h"

namespace nsa {
// ------------------------------------------------------------------ stores

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
template <class O>
__device__ __forceinline__ f32x4 load4(const typename O::storage* p);
template <>
__device__ __forceinline__ f32x4 load4<BF16>(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
}
template <>
__device__ __forceinline__ f32x4 load4<F32>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// The block means of K enter the block scores, and the selection is judged
// against exact means: with bf16 operands the mean is carried as a high part
// plus a bf16 low part (hi + lo holds ~16 significant bits), and every
// compressed-branch QK product is the sum of two MFMAs.
template <class T>
constexpr bool kSplitKc = false;
template <>
constexpr bool kSplitKc<BF16> = true;

// Tiles in the compressed kernel's LDS stage: two buffers of K and V, plus
// the low part of K when the means are split and LOL (low part through LDS)
// is chosen; otherwise each wave reads the low part from L2 itself.
template <class T, bool LOL>
constexpr int cmp_stage_tiles() {
  return kSplitKc<T> && LOL ? 6 : 4;
}

// Sequence b's context length and first query position (the uniform L and
// t0 unless per-sequence arrays are given). A pair outside 0 <= t0 <= L <=
// a.L gives an empty sequence: no query rows, no key rows.
struct SeqSpan {
  int L, t0;
};
__device__ __forceinline__ SeqSpan seq_span(const PrefillArgs& a, int b) {
  if (a.seq_lens == nullptr) return SeqSpan{a.L, a.t0};
  const int L = a.seq_lens[b], t0 = a.q_offs != nullptr ? a.q_offs[b] : 0;
  if (L < 0 || L > a.L || t0 < 0 || t0 > L) return SeqSpan{0, 0};
  return SeqSpan{L, t0};
}

// ------------------------------------------------------------------ k_prep

template <class T, int D>
__global__ __launch_bounds__(256) void k_prep(PrefillArgs a) {
  using S = typename T::storage;
  __shared__ __align__(16) S kbuf[64 * D];
  __shared__ __align__(16) S vbuf[64 * D];
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int Lb = __builtin_amdgcn_readfirstlane(seq_span(a, b).L);  // key rows past it are zero-filled
  const bool have = j < a.Nb;
  if (have) {
    const S* K = static_cast<const S*>(a.k) + b * a.ks[0] + g * a.ks[2];
    const S* V = static_cast<const S*>(a.v) + b * a.vs[0] + g * a.vs[2];
    constexpr int VPR = D / 8;
    for (int e = tid; e < 64 * VPR; e += 256) {
      const int r = e / VPR, c = (e % VPR) * 8;
      const int t = j * 64 + r;
      Frag<T> kf = frag_zero<T>(), vf = frag_zero<T>();
      if (t < Lb) {
        kf = frag_load<T>(K + static_cast<int64_t>(t) * a.ks[1] + c);
        vf = frag_load<T>(V + static_cast<int64_t>(t) * a.vs[1] + c);
      }
      frag_store<T>(kbuf + r * D + c, kf);
      frag_store<T>(vbuf + r * D + c, vf);
    }
  }
  __syncthreads();
  if (have) {
    const int64_t tile = (static_cast<int64_t>(b * a.G + g) * a.Nb + j) * (64 * D);
    S* kt = static_cast<S*>(a.kt) + tile;
    S* vt = static_cast<S*>(a.vt) + tile;
    constexpr int NF = 8 * D;  // fragments per 64 x D tile
    for (int f = tid; f < NF; f += 256) {
      const int lane = f & 63;
      const int ks_ = f >> 6;
      const int kt_i = ks_ / (D / 32), s = ks_ % (D / 32);
      frag_store<T>(kt + f * 8,
                    frag_load<T>(kbuf + (16 * kt_i + (lane & 15)) * D + 32 * s + 8 * (lane >> 4)));
      const int dt = ks_ >> 1, sv = ks_ & 1;
      const int dcol = 16 * dt + (lane & 15), a4 = lane >> 4;
      __align__(16) S tmp[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int key = 32 * sv + (jj < 4 ? 4 * a4 + jj : 16 + 4 * a4 + (jj - 4));
        tmp[jj] = vbuf[key * D + dcol];
      }
      frag_store<T>(vt + f * 8, frag_load<T>(tmp));
    }
  }
  if (j < a.NcT * 64) {
    const int c = j >> 6, r = j & 63;
    const int64_t tile = (static_cast<int64_t>(b * a.G + g) * a.NcT + c) * (64 * D);
    S* kc = static_cast<S*>(a.kct) + tile;
    S* vc = static_cast<S*>(a.vct) + tile;
    S* kcl = kSplitKc<T> ? static_cast<S*>(a.kclt) + tile : nullptr;
    for (int d = tid; d < D; d += 256) {
      float sk = 0.f, sv = 0.f;
      if (j < a.Nc) {
        for (int i = 0; i < 64; ++i) {
          sk += to_f32<T>(kbuf[i * D + d]);
          sv += to_f32<T>(vbuf[i * D + d]);
        }
        sk *= (1.0f / 64.0f);
        sv *= (1.0f / 64.0f);
      }
      const S hi = from_f32<T>(sk);
      kc[ktile_off(r, d, D)] = hi;
      if (kSplitKc<T>) kcl[ktile_off(r, d, D)] = from_f32<T>(sk - to_f32<T>(hi));
      vc[vtile_off(r, d)] = from_f32<T>(sv);
    }
  }
}

// ------------------------------------------------------------------ shared pieces

// Cooperative copy of one or two 64 x D tiles (fragment-major, contiguous)
// from global memory into LDS through registers: issue() starts the loads of
// the next tiles, commit() stores them once the current tiles are consumed.
template <class T, int D, int NT>
struct TileStager {
  static constexpr int kVec = 64 * D * static_cast<int>(sizeof(typename T::storage)) / 16;
  static constexpr int kPer = kVec / NT;
  u32x4 r[3][kPer];
  __device__ __forceinline__ void issue(const void* a, const void* b, const void* c, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) r[0][i] = static_cast<const u32x4*>(a)[tid + NT * i];
    if (b != nullptr) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) r[1][i] = static_cast<const u32x4*>(b)[tid + NT * i];
    }
    if (c != nullptr) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) r[2][i] = static_cast<const u32x4*>(c)[tid + NT * i];
    }
  }
  __device__ __forceinline__ void commit(void* a, void* b, void* c, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) static_cast<u32x4*>(a)[tid + NT * i] = r[0][i];
    if (b != nullptr) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) static_cast<u32x4*>(b)[tid + NT * i] = r[1][i];
    }
    if (c != nullptr) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) static_cast<u32x4*>(c)[tid + NT * i] = r[2][i];
    }
  }
};

// ------------------------------------------------------------------ k_cmpwin

template <class T, class O, int D, int NW, bool LOL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_cmpwin(PrefillArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int TPW = kCmpTPW, KS = D / 32, DT = D / 16, NT = 64 * NW, TILE = 64 * D;
  constexpr bool LOLDS = kSplitKc<T> && LOL;
  constexpr int BUF = cmp_stage_tiles<T, LOL>() / 2 * TILE;  // elements of one stage buffer
  extern __shared__ __align__(16) unsigned char smem[];
  // [2 buffers][K, V (, K low part)][TILE], then the block scores; the top-k
  // scratch reuses the stage once the compressed passes are done
  S* stage = reinterpret_cast<S*>(smem);
  const int NcPad = a.NcT * 64;
  float* scb = reinterpret_cast<float*>(smem + 2 * BUF * sizeof(S));
  uint64_t* survb = reinterpret_cast<uint64_t*>(smem);
  int* selbb = reinterpret_cast<int*>(survb + NW * kSurvCap);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int BG = a.B * a.G;
  const int tile = a.cmp_tiles - 1 - static_cast<int>(blockIdx.x) / BG;  // heaviest first
  const int bg = static_cast<int>(blockIdx.x) % BG, b = bg / a.G, g = bg % a.G;
  const SeqSpan sp = seq_span(a, b);
  const int t0q = __builtin_amdgcn_readfirstlane(sp.t0);  // first query position; query row = position - t0q
  const int Le = __builtin_amdgcn_readfirstlane(min(sp.L, sp.t0 + a.Lq));  // end of the query positions
  const int T0 = t0q + tile * TPW * NW;   // absolute position of the workgroup's first token
  if (T0 >= Le) return;                   // whole workgroup
  const int col = lane & 15, grp = lane >> 4;
  const bool colv = col < a.Hg;
  const int h = g * a.Hg + col;
  const int tw = T0 + TPW * wave;                     // this wave's first token
  const int Tl = min(T0 + TPW * NW - 1, Le - 1);     // the workgroup's last token
  const float sl2 = a.scale_log2;
  const int64_t bgoff = static_cast<int64_t>(b * a.G + g);

  const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + h * a.qs[2] + 8 * grp;
  const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0] + h * a.gs[2];
  Frag<T> qf[TPW][KS];
  float gcmp[TPW], gwin[TPW];
  int nvis[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = tw + qt;
    const bool valid = t < Le && colv;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = valid ? frag_load<T>(Q + static_cast<int64_t>(t - t0q) * a.qs[1] + 32 * s) : frag_zero<T>();
    gcmp[qt] = valid ? to_f32<T>(GT[static_cast<int64_t>(t - t0q) * a.gs[1]]) : 0.f;
    gwin[qt] = valid ? to_f32<T>(GT[static_cast<int64_t>(t - t0q) * a.gs[1] + 2]) : 0.f;
    nvis[qt] = t < Le ? (t + 1) >> 6 : 0;
  }
  f32x4 oacc[TPW][DT];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  TileStager<T, D, NT> stg;

  // ---- sliding window over the workgroup's band of key blocks
  {
    const S* KT = static_cast<const S*>(a.kt) + bgoff * a.Nb * TILE;
    const S* VT = static_cast<const S*>(a.vt) + bgoff * a.Nb * TILE;
    const int b0 = max(0, T0 - a.w + 1) >> 6, b1 = Tl >> 6;
    float mw[TPW], lw[TPW];
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      mw[qt] = kNegBig;
      lw[qt] = 0.f;
    }
    stg.issue(KT + static_cast<int64_t>(b0) * TILE, VT + static_cast<int64_t>(b0) * TILE, nullptr, tid);
    stg.commit(stage, stage + TILE, nullptr, tid);
    __syncthreads();
    // INNER: both halves of the block lie inside the window of every token of
    // the workgroup (no band test, no masks); the band's edge blocks take
    // the general body. Three loops, so each body is straight-line code.
    auto stepw = [&](auto inner_c, int blk) __attribute__((always_inline)) {
      constexpr bool INNER = decltype(inner_c)::value;
      const int buf = (blk - b0) & 1;
      const bool more = blk < b1;
      if (more)
        stg.issue(KT + static_cast<int64_t>(blk + 1) * TILE, VT + static_cast<int64_t>(blk + 1) * TILE, nullptr,
                  tid);
      const S* kt = stage + buf * BUF;
      const S* vt = kt + TILE;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kb = 64 * blk + 32 * s2;
        if (!INNER && (kb > tw + TPW - 1 || kb + 31 < tw - a.w + 1)) continue;  // outside this wave's band
        Frag<T> kf[2][KS];
        Frag<T> vf[DT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int s = 0; s < KS; ++s) kf[h2][s] = frag_load<T>(kt + ktile_frag(2 * s2 + h2, s, lane, D));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vt + vtile_frag(dt, s2, lane));
        // all 32 keys inside every token's window: no masks needed
        const bool full = INNER || (kb >= tw + TPW - a.w && kb + 31 <= tw && tw + TPW - 1 < Le);
#pragma unroll
        for (int qt = 0; qt < TPW; ++qt) {
          const int t = tw + qt;
          f32x4 st[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            st[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) mma(st[h2], kf[h2][s], qf[qt][s]);
          }
          if (full)
            online_step<T, DT, false>(st, kb, 0, 0, grp, sl2, mw[qt], lw[qt], oacc[qt], vf);
          else
            online_step<T, DT, true>(st, kb, t - a.w + 1, t < Le ? t : -1, grp, sl2, mw[qt], lw[qt],
                                     oacc[qt], vf);
        }
      }
      if (more) stg.commit(stage + (buf ^ 1) * BUF, stage + (buf ^ 1) * BUF + TILE, nullptr, tid);
      __syncthreads();
    };
    // inner blocks: 64 blk >= (last token + 1) - w and 64 blk + 63 <= first token
    int lo = b1 + 1, hi = b1;
    if (T0 + TPW * NW - 1 < Le) {
      const int x = T0 + TPW * NW - a.w;  // lowest first key of an inner block
      lo = x <= 0 ? b0 : max(b0, (x + 63) >> 6);
      hi = T0 >= 63 ? min(b1, (T0 - 63) >> 6) : -1;
      if (lo > hi) lo = hi + 1;
    }
    int blk = b0;
    for (; blk < lo && blk <= b1; ++blk) stepw(std::integral_constant<bool, false>{}, blk);
    for (; blk <= hi; ++blk) stepw(std::integral_constant<bool, true>{}, blk);
    for (; blk <= b1; ++blk) stepw(std::integral_constant<bool, false>{}, blk);
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const float lt = col_sum4(lw[qt]);
      const float f = lt > 0.f ? gwin[qt] / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] *= f;
    }
  }

  // ---- compressed branch
  const int nch = (((Tl + 1) >> 6) + 63) >> 6;
  const S* KC = static_cast<const S*>(a.kct) + bgoff * a.NcT * TILE;
  const S* KCL = kSplitKc<T> ? static_cast<const S*>(a.kclt) + bgoff * a.NcT * TILE : nullptr;
  const S* VC = static_cast<const S*>(a.vct) + bgoff * a.NcT * TILE;

  // pass 1: log-sum-exp (log2 domain) from the high part of the block means.
  // An error e_h in a head's log-sum-exp scales all of that head's
  // probabilities by exp(-e_h); the differences between block scores, which
  // the selection compares, move only in second order. Pass 2 uses the full
  // precision logits.
  float m[TPW], ls[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    m[qt] = kNegBig;
    ls[qt] = 0.f;
  }
  if (nch > 0) {
    stg.issue(KC, nullptr, nullptr, tid);
    stg.commit(stage, nullptr, nullptr, tid);
    __syncthreads();
  }
  // Fully visible chunks first, then the partial ones, each loop one
  // straight-line body (FULL drops the masks).
  auto step1 = [&](auto full_c, int c) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) stg.issue(KC + static_cast<int64_t>(c + 1) * TILE, nullptr, nullptr, tid);
    const S* kc = stage + buf * BUF;
    f32x4 st[TPW][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      Frag<T> kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = frag_load<T>(kc + ktile_frag(kt, s, lane, D));
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
        st[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(st[qt][kt], kf[s], qf[qt][s]);
      }
    }
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      // maximum over the raw scores (sl2 > 0); the scaling goes into the exponent
      float lmx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (FULL || 64 * c + 16 * kt + 4 * grp + i < nvis[qt]) ? st[qt][kt][i] : -INFINITY;
          st[qt][kt][i] = x;
          lmx = fmaxf(lmx, x);
        }
      lmx = fmaxf(lmx * sl2, kNegBig);
      if (wave_any(lmx > m[qt] + kLazyMax)) {
        const float mn = fmaxf(m[qt], col_max4(lmx));
        ls[qt] *= fast_exp2(m[qt] - mn);
        m[qt] = mn;
      }
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += fast_exp2(fmaf(st[qt][kt][i], sl2, -m[qt]));
      ls[qt] += sum;
    }
    if (more) stg.commit(stage + (buf ^ 1) * BUF, nullptr, nullptr, tid);
    __syncthreads();
  };
  // chunks [0, nfull) are visible to both tokens in full
  const int nfull = __builtin_amdgcn_readfirstlane(min(nch, nvis[0] >> 6));
  {
    int c = 0;
    for (; c < nfull; ++c) step1(std::integral_constant<bool, true>{}, c);
    for (; c < nch; ++c) step1(std::integral_constant<bool, false>{}, c);
  }
  float lse2[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const float tot = col_sum4(ls[qt]);
    lse2[qt] = (nvis[qt] > 0 && colv) ? m[qt] + fast_log2(tot) : INFINITY;
  }

  // pass 2: probabilities, gate_cmp * P . Vc into the accumulators, block scores
  float* sc = scb + static_cast<size_t>(wave) * TPW * NcPad;
  if (nch > 0) {
    stg.issue(KC, VC, LOLDS ? KCL : nullptr, tid);
    stg.commit(stage, stage + TILE, LOLDS ? stage + 2 * TILE : nullptr, tid);
    __syncthreads();
  }
  // One 64-key chunk; FULL: every key visible to both tokens (no masks).
  // The full chunks come first and run as one loop, the partial ones as a
  // second: each loop body is straight-line code (no branch between the QK
  // products, the softmax and the PV products) that the compiler schedules
  // as one region. The block scores are computed even when the caller
  // injects the selection (they are then unused).
  auto chunk2 = [&](auto full_c, int c, const S* kc, const S* vc, const S* kcl) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f32x4 st[TPW][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        Frag<T> kf[KS], kl[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          kf[s] = frag_load<T>(kc + ktile_frag(2 * s2 + h2, s, lane, D));
          if (kSplitKc<T>) kl[s] = frag_load<T>(kcl + ktile_frag(2 * s2 + h2, s, lane, D));
        }
#pragma unroll
        for (int qt = 0; qt < TPW; ++qt) {
          st[qt][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            mma(st[qt][h2], kf[s], qf[qt][s]);
            if (kSplitKc<T>) mma(st[qt][h2], kl[s], qf[qt][s]);
          }
        }
      }
      Frag<T> vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vc + vtile_frag(dt, s2, lane));
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(st[qt][h2][i] * sl2 - lse2[qt]);
            st[qt][h2][i] = (FULL || 64 * c + 32 * s2 + 16 * h2 + 4 * grp + i < nvis[qt]) ? p : 0.f;
          }
        {
          // the head sum of key 16·c₃ + 4·grp + 2·c₀ + c₁ of this half (c = col)
          const float r = row_scatter_sum8(st[qt], col);
          sc[qt * NcPad + 64 * c + 32 * s2 + 16 * ((col >> 3) & 1) + 4 * grp + 2 * (col & 1) + ((col >> 1) & 1)] = r;
        }
        const Frag<T> pf = pack_p<T>(st[qt][0] * gcmp[qt], st[qt][1] * gcmp[qt]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) mma(oacc[qt][dt], vf[dt], pf);
      }
    }
  };
  auto step2 = [&](auto full_c, int c) __attribute__((always_inline)) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more)
      stg.issue(KC + static_cast<int64_t>(c + 1) * TILE, VC + static_cast<int64_t>(c + 1) * TILE,
                LOLDS ? KCL + static_cast<int64_t>(c + 1) * TILE : nullptr, tid);
    const S* kc = stage + buf * BUF;
    const S* vc = kc + TILE;
    // low parts (bf16 inputs only): staged after V, or read from L2
    const S* kcl = LOLDS ? vc + TILE : kSplitKc<T> ? KCL + static_cast<int64_t>(c) * TILE : nullptr;
    chunk2(full_c, c, kc, vc, kcl);
    if (more)
      stg.commit(stage + (buf ^ 1) * BUF, stage + (buf ^ 1) * BUF + TILE,
                 LOLDS ? stage + (buf ^ 1) * BUF + 2 * TILE : nullptr, tid);
    __syncthreads();
  };
  int c = 0;
  for (; c < nfull; ++c) step2(std::integral_constant<bool, true>{}, c);
  for (; c < nch; ++c) step2(std::integral_constant<bool, false>{}, c);

  // ---- gate_win * O_win + gate_cmp * O_cmp -> out (k_sel adds the selected branch)
  {
    SO* OUT = static_cast<SO*>(a.out) + b * a.os[0] + h * a.os[2] + 4 * grp;
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = tw + qt;
      if (t < Le && colv) {
        SO* o = OUT + static_cast<int64_t>(t - t0q) * a.os[1];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4<O>(o + 16 * dt, oacc[qt][dt]);
      }
    }
  }

  // ---- selection
  if (!a.inject) {
    wave_lds_sync();
    uint64_t* surv = survb + static_cast<size_t>(wave) * kSurvCap;
    int* selb = selbb + wave * 64;
#pragma unroll 1
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = tw + qt;
      if (t >= Le) break;
      int32_t* row = a.idx + ((static_cast<int64_t>(b) * a.Lq + (t - t0q)) * a.G + g) * a.n;
      topk_wave(sc + qt * NcPad, t >> 6, a.n, row, surv, selb, lane);
    }
  }
}

// ------------------------------------------------------------------ k_sel

// Registers of one 32-key half block: K fragments of its two key tiles and
// the V^T fragments of its k-step.
template <class T, int D>
struct HalfBlock {
  Frag<T> k[2][D / 32];
  Frag<T> v[D / 16];
};

template <class T, int D>
__device__ __forceinline__ void half_load(HalfBlock<T, D>& hb, const typename T::storage* KT,
                                          const typename T::storage* VT, int j, int hh, int lane) {
  const typename T::storage* kt = KT + static_cast<int64_t>(j) * (64 * D);
  const typename T::storage* vt = VT + static_cast<int64_t>(j) * (64 * D);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) hb.k[h2][s] = frag_load<T>(kt + ktile_frag(2 * hh + h2, s, lane, D));
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) hb.v[dt] = frag_load<T>(vt + vtile_frag(dt, hh, lane));
}

template <class T, int D, bool MASK>
__device__ __forceinline__ void half_attend(const HalfBlock<T, D>& hb, const Frag<T> (&qf)[D / 32],
                                            int kb, int t, int grp, float sl2, float& m, float& l,
                                            f32x4 (&acc)[D / 16]) {
  f32x4 st[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    st[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) mma(st[h2], hb.k[h2][s], qf[s]);
  }
  online_step<T, D / 16, MASK>(st, kb, 0, t, grp, sl2, m, l, acc, hb.v);
}

// A wave owns kSelTPW consecutive tokens of one KV group. The half blocks
// they selected are marked in a per-wave LDS bitmap (one byte per half
// block, bit qt = token qt uses it) and compacted into a step list in
// ascending block order: a half block chosen by several of the wave's tokens
// (always the own block, shared by neighbouring tokens) is loaded once, and
// every wave sweeps the blocks in the same direction, so concurrent gathers
// stay closer together in L2. The steps stream through a ring of kSelRing
// half-block register buffers; each step runs the online-softmax update of
// every token in its mask. Query fragments are kept in LDS.
template <class T, class O, int D, bool SAVE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_sel(PrefillArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int TPW = kSelTPW, NB = kSelRing, KS = D / 32, DT = D / 16;
  constexpr int FE = sizeof(Frag<T>) / 16;  // 16-byte words per fragment lane
  __shared__ u32x4 q_lds[4][TPW][KS][FE][64];
  extern __shared__ __align__(16) unsigned char sel_dyn[];  // per wave: bitmap words, then steps
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // This workgroup's (group, sequence, tile); workgroup i runs on XCD i % 8.
  // Contiguous: each XCD takes an eighth of the (group, sequence, tile)
  // items in order, so an XCD serves one group, and for a whole prefill the
  // XCD with the early tokens works from a small set of blocks (the best L2
  // hit rate, measured). Interleaved (when G divides 8): each group is served
  // by 8 / G XCDs that take its tiles in turn (k, k + 8/G, ...), sequence
  // after sequence, so those XCDs get equal shares of every sequence whatever
  // the lengths (for varlen batches and chunks, measured faster). There are
  // no workgroup barriers in this kernel, so workgroups without an item exit.
  int g, b, tile;
  {
    const int xcd = static_cast<int>(blockIdx.x & 7), slot = static_cast<int>(blockIdx.x >> 3);
    if (a.sel_interleave) {
      const int pg = 8 / a.G, k = xcd % pg;  // a group's XCDs are neighbours: xcd / pg = g
      const int tk = (a.sel_tiles - k + pg - 1) / pg;  // this XCD's tiles of one sequence
      if (slot >= a.B * tk) return;
      g = xcd / pg;
      b = slot / tk;
      tile = k + pg * (slot % tk);
    } else if (a.sel_bounds[0] >= 0) {
      const int pg = 8 / a.G, k = xcd % pg;
      const int item = a.sel_bounds[k] + slot;
      if (item >= a.sel_bounds[k + 1]) return;
      g = xcd / pg;
      b = item / a.sel_tiles;
      tile = item % a.sel_tiles;
    } else {
      const int N = a.B * a.G * a.sel_tiles;
      const int item = xcd * ((N + 7) >> 3) + slot;
      if (item >= N) return;
      g = item / (a.B * a.sel_tiles);
      const int rem = item % (a.B * a.sel_tiles);
      b = rem / a.sel_tiles;
      tile = rem % a.sel_tiles;
    }
  }
  const SeqSpan sp = seq_span(a, b);
  const int t0q = __builtin_amdgcn_readfirstlane(sp.t0);  // first query position; query row = position - t0q
  const int Le = __builtin_amdgcn_readfirstlane(min(sp.L, sp.t0 + a.Lq));  // end of the query positions
  const int t0 = t0q + (tile * 4 + wave) * TPW;  // absolute position of the wave's first token
  if (t0 >= Le) return;
  const int col = lane & 15, grp = lane >> 4;
  const bool colv = col < a.Hg;
  const int h = g * a.Hg + col;
  const float sl2 = a.scale_log2;
  const int64_t tb = static_cast<int64_t>(b * a.G + g) * a.Nb * (64 * D);
  const S* KT = static_cast<const S*>(a.kt) + tb;
  const S* VT = static_cast<const S*>(a.vt) + tb;
  const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + h * a.qs[2] + 8 * grp;
  const int n = a.n;
  uint32_t* bm = reinterpret_cast<uint32_t*>(sel_dyn) + static_cast<size_t>(wave) * (a.sel_bm_words + TPW * 128);
  int* steps = reinterpret_cast<int*>(bm + a.sel_bm_words);

  // ---- query fragments -> LDS; the wave's half blocks -> bitmap -> step list
  const int tl = min(t0 + TPW - 1, Le - 1);
  const int nwords = (2 * ((tl >> 6) + 1) + 3) >> 2;  // half blocks 0 .. 2 own(tl) + 1
  for (int w = lane; w < nwords; w += 64) bm[w] = 0u;
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    const bool tv = t < Le;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Frag<T> f =
          (tv && colv) ? frag_load<T>(Q + static_cast<int64_t>(t - t0q) * a.qs[1] + 32 * s) : frag_zero<T>();
      const u32x4* w = reinterpret_cast<const u32x4*>(&f);
#pragma unroll
      for (int e = 0; e < FE; ++e) q_lds[wave][qt][s][e][lane] = w[e];
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    if (t >= Le) break;
    const int own = t >> 6;
    const int32_t* row = a.idx + ((static_cast<int64_t>(b) * a.Lq + (t - t0q)) * a.G + g) * n;
    const int j = lane < n ? row[lane] : -1;
    if (j >= 0 && j <= own) {  // padding / unusable injected entries drop out
      const uint32_t bit = 1u << qt;
      atomicOr(&bm[j >> 1], bit << (16 * (j & 1)));
      if (64 * j + 32 <= t) atomicOr(&bm[j >> 1], bit << (16 * (j & 1) + 8));
    }
  }
  wave_lds_sync();
  int nsteps = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int w0 = 0; w0 < nwords; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t word = w < nwords ? bm[w] : 0u;
    int cnt = 0;
#pragma unroll
    for (int by = 0; by < 4; ++by) cnt += ((word >> (8 * by)) & 0xFFu) != 0u;
    // prefix sum of the per-lane counts (0..4) over lower lanes, bit by bit
    int pos = nsteps;
    int tot = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
      const uint64_t bal = __ballot((cnt >> bit) & 1);
      pos += __popcll(bal & below) << bit;
      tot += __popcll(bal) << bit;
    }
#pragma unroll
    for (int by = 0; by < 4; ++by) {
      const uint32_t msk = (word >> (8 * by)) & 0xFFu;
      if (msk != 0u) {
        const int hb = 4 * w + by;  // half block: block hb / 2, half hb % 2
        steps[pos++] = (hb >> 1) | ((hb & 1) << 23) | static_cast<int>(msk << 24);
      }
    }
    nsteps += tot;
  }
  wave_lds_sync();

  float m[TPW], l[TPW];
  f32x4 acc[TPW][DT];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    m[qt] = kNegBig;
    l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // The ring is loaded unconditionally -- a step past the end reloads the
  // last step's half block and is run with no tokens -- and the loop's only
  // exit is at its top, so the count of loads in flight is the same on every
  // path and each step waits only for its own slot's loads while the other
  // slots' stay in flight.
  if (nsteps > 0) {
    HalfBlock<T, D> ring[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int code = steps[min(k, nsteps - 1)];
      half_load<T, D>(ring[k], KT, VT, code & 0x7FFFFF, (code >> 23) & 1, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll 1
    for (int base = 0; base < nsteps; base += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int s = base + k;
        const int code = steps[min(s, nsteps - 1)];
        const int j = code & 0x7FFFFF, hh = (code >> 23) & 1;
        const int msk = s < nsteps ? static_cast<int>(static_cast<uint32_t>(code) >> 24) : 0;
        const int kb = 64 * j + 32 * hh;
#pragma unroll
        for (int qt = 0; qt < TPW; ++qt) {
          if ((msk >> qt) & 1) {
            const int t = t0 + qt;
            Frag<T> qf[KS];
#pragma unroll
            for (int ss = 0; ss < KS; ++ss) {
              u32x4* w = reinterpret_cast<u32x4*>(&qf[ss]);
#pragma unroll
              for (int e = 0; e < FE; ++e) w[e] = q_lds[wave][qt][ss][e][lane];
            }
            if (kb + 31 <= t)
              half_attend<T, D, false>(ring[k], qf, kb, t, grp, sl2, m[qt], l[qt], acc[qt]);
            else
              half_attend<T, D, true>(ring[k], qf, kb, t, grp, sl2, m[qt], l[qt], acc[qt]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        const int nc = steps[min(s + NB, nsteps - 1)];
        half_load<T, D>(ring[k], KT, VT, nc & 0x7FFFFF, (nc >> 23) & 1, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0] + h * a.gs[2];
  SO* OUT = static_cast<SO*>(a.out) + b * a.os[0] + h * a.os[2] + 4 * grp;
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    const float lt = col_sum4(l[qt]);
    if (t < Le && colv) {
      const float gsl = to_f32<T>(GT[static_cast<int64_t>(t - t0q) * a.gs[1] + 1]);
      const float f = lt > 0.f ? gsl / lt : 0.f;
      SO* o = OUT + static_cast<int64_t>(t - t0q) * a.os[1];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 prev = load4<O>(o + 16 * dt);
        store4<O>(o + 16 * dt, prev + acc[qt][dt] * f);
      }
      if (SAVE) {  // the branch's own output and log-sum-exp, kept for the backward pass
        const int64_t r = (static_cast<int64_t>(b) * a.Lq + (t - t0q)) * a.Hq + h;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        SO* so = static_cast<SO*>(a.save_o) + r * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4<O>(so + 16 * dt, acc[qt][dt] * inv);
        if (grp == 0) a.save_lse[r] = lt > 0.f ? (m[qt] + fast_log2(lt)) * kLn2 : -INFINITY;
      }
    }
  }
}

size_t sel_lds_bytes(int Nb, int D, bool bf16) {
  const size_t need = 4 * (static_cast<size_t>(sel_bm_words(Nb)) + kSelTPW * 128) * sizeof(uint32_t);
  const size_t stat = sel_static_lds_bytes(D, bf16);
  const size_t cap = kSelLdsOneWg > stat ? kSelLdsOneWg - stat : 0;  // total > half a CU's LDS
  return need > cap ? need : cap;
}

size_t cmpwin_lds_bytes(int waves, int NcT, int D, bool bf16, bool lo_lds) {
  const int tiles = bf16 ? (lo_lds ? cmp_stage_tiles<BF16, true>() : cmp_stage_tiles<BF16, false>())
                         : cmp_stage_tiles<F32, false>();
  const size_t stage = tiles * 64 * static_cast<size_t>(D) * (bf16 ? 2 : 4);
  const size_t topk = static_cast<size_t>(waves) * cmp_topk_scratch_bytes();
  return (stage > topk ? stage : topk) + cmp_lds_bytes(waves, NcT);
}

static hipError_t record(hipEvent_t* ev, int i, hipStream_t st) {
  return ev != nullptr ? hipEventRecord(ev[i], st) : hipSuccess;
}

template <class T, class O, int D, int NW, bool LOL>
static hipError_t launch_cmpwin(const PrefillArgs& a, hipStream_t st) {
  const size_t lds = cmpwin_lds_bytes(NW, a.NcT, D, sizeof(typename T::storage) == 2, LOL);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cmpwin<T, O, D, NW, LOL>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_cmpwin<T, O, D, NW, LOL>), dim3(a.B * a.G * a.cmp_tiles), dim3(64 * NW), lds, st, a);
  return hipSuccess;
}

template <class T, class O, int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st, hipEvent_t* ev) {
  hipError_t e;
  const int nblk_prep = max(a.Nb, a.NcT * 64);
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_prep<T, D>), dim3(nblk_prep, a.G, a.B), dim3(256), 0, st, a);
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  if (a.cmp_waves == 8) {
    if (a.cmp_lo_lds) e = launch_cmpwin<T, O, D, 8, true>(a, st);
    else e = launch_cmpwin<T, O, D, 8, false>(a, st);
  } else if (a.cmp_waves == 4) {
    e = launch_cmpwin<T, O, D, 4, false>(a, st);
  } else if (a.cmp_waves == 2) {
    e = launch_cmpwin<T, O, D, 2, false>(a, st);
  } else {
    e = launch_cmpwin<T, O, D, 1, false>(a, st);
  }
  if (e != hipSuccess) return e;
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
  // workgroups per XCD (see the item mapping in k_sel)
  int per = a.sel_interleave ? a.B * ((a.sel_tiles + 8 / a.G - 1) / (8 / a.G)) : (a.B * a.G * a.sel_tiles + 7) / 8;
  if (!a.sel_interleave && a.sel_bounds[0] >= 0) {
    per = 0;
    for (int k = 0; k < 8 / a.G; ++k) per = max(per, a.sel_bounds[k + 1] - a.sel_bounds[k]);
  }
  // Static + dynamic LDS above half a CU's caps residency at one workgroup
  // (4 waves) per CU, which was measured faster (~13 % at 64k) than two: the
  // gathers then contend less for L2.
  const size_t sel_lds = sel_lds_bytes(a.Nb, D, sizeof(typename T::storage) == 2);
  if (a.save_o != nullptr) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sel<T, O, D, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sel_lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_sel<T, O, D, true>), dim3(per * 8), dim3(256), sel_lds, st, a);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sel<T, O, D, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sel_lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_sel<T, O, D, false>), dim3(per * 8), dim3(256), sel_lds, st, a);
  }
  if ((e = record(ev, 3, st)) != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, bool out_bf16, hipStream_t st,
                          hipEvent_t* ev) {
  if (in_bf16) {
    if (out_bf16)
      return a.D == 64 ? launch_prefill_t<BF16, BF16, 64>(a, st, ev)
                       : launch_prefill_t<BF16, BF16, 128>(a, st, ev);
    return a.D == 64 ? launch_prefill_t<BF16, F32, 64>(a, st, ev)
                     : launch_prefill_t<BF16, F32, 128>(a, st, ev);
  }
  return a.D == 64 ? launch_prefill_t<F32, F32, 64>(a, st, ev) : launch_prefill_t<F32, F32, 128>(a, st, ev);
}

}  // namespace nsa
