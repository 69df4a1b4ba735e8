// NSA prefill on gfx950: three kernels per call.
//
//  k_prep  block compression + re-layout. One workgroup per 64-token block
//          (b, g, j): the block's K and V are staged in LDS, written back as a
//          fragment-major K tile and a permuted V^T tile, and, for complete
//          blocks, their fp32 means (the compressed keys/values) are written
//          into the compressed tiles. Compression by block means, stride 64:
//          compressed block representations, NSA factory write-up
//          (chencunli.com), section "What dynamic sparsity actually
//          sparsifies"; block size from the NSA how-to (qwbw.cn/news/106443),
//          section 3.
//  k_cmp   compressed branch + block scores + top-k selection. A wave owns 4
//          query tokens of one KV group (16 query heads each). Pass 1 finds the
//          log-sum-exp of the compressed logits; pass 2 recomputes them, forms
//          normalised probabilities, accumulates the compressed output with
//          MFMA and the per-block scores (probabilities summed over the
//          group's heads, a DPP row reduction) into LDS; then the wave selects
//          the blocks. Writes gate_cmp * O_cmp into out and the selection into
//          idx. Workgroups run heaviest (latest tokens) first.
//  k_sw    selected-block branch + sliding-window branch + gate combination.
//          A wave owns 2 tokens: the window band is shared by both, the
//          selected blocks are gathered per token straight from the K/V tiles
//          in MFMA-fragment order. out += gate_slc * O_slc + gate_win * O_win.
//          Work items are grouped by KV group per XCD so each XCD's L2 serves
//          one group's K/V.
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
  w.x = f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16);
  w.y = f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16);
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

// ------------------------------------------------------------------ k_prep

template <class T, int D>
__global__ __launch_bounds__(256) void k_prep(PrefillArgs a) {
  using S = typename T::storage;
  __shared__ __align__(16) S kbuf[64 * D];
  __shared__ __align__(16) S vbuf[64 * D];
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const bool have = j < a.Nb;
  if (have) {
    const S* K = static_cast<const S*>(a.k) + b * a.ks[0] + g * a.ks[2];
    const S* V = static_cast<const S*>(a.v) + b * a.vs[0] + g * a.vs[2];
    constexpr int VPR = D / 8;
    for (int e = tid; e < 64 * VPR; e += 256) {
      const int r = e / VPR, c = (e % VPR) * 8;
      const int t = j * 64 + r;
      Frag<T> kf = frag_zero<T>(), vf = frag_zero<T>();
      if (t < a.L) {
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

// ------------------------------------------------------------------ k_cmp

template <class T, class O, int D, int TPW>
__global__ __launch_bounds__(256) void k_cmp(PrefillArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int KS = D / 32, DT = D / 16;
  extern __shared__ __align__(16) unsigned char smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int BG = a.B * a.G;
  const int tile = a.cmp_tiles - 1 - static_cast<int>(blockIdx.x) / BG;  // heaviest first
  const int bg = static_cast<int>(blockIdx.x) % BG, b = bg / a.G, g = bg % a.G;
  const int t0 = (tile * nw + wave) * TPW;
  if (t0 >= a.L) return;  // no workgroup barriers below
  const int col = lane & 15, grp = lane >> 4;
  const bool colv = col < a.Hg;
  const int h = g * a.Hg + col;
  const int NcPad = a.NcT * 64;

  const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + h * a.qs[2] + 8 * grp;
  Frag<T> qf[TPW][KS];
  int nvis[TPW];
  int nvmax = 0;
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    const bool valid = t < a.L;
    nvis[qt] = valid ? (t + 1) >> 6 : 0;
    nvmax = max(nvmax, nvis[qt]);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = (valid && colv) ? frag_load<T>(Q + static_cast<int64_t>(t) * a.qs[1] + 32 * s)
                                  : frag_zero<T>();
  }
  const int nch = (nvmax + 63) >> 6;
  const int64_t tbase = static_cast<int64_t>(b * a.G + g) * a.NcT * (64 * D);
  const S* KC = static_cast<const S*>(a.kct) + tbase;
  const S* KCL = kSplitKc<T> ? static_cast<const S*>(a.kclt) + tbase : nullptr;
  const S* VC = static_cast<const S*>(a.vct) + tbase;
  const float sl2 = a.scale_log2;

  // ---- pass 1: log-sum-exp of the visible compressed logits (log2 domain)
  float m[TPW], ls[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    m[qt] = kNegBig;
    ls[qt] = 0.f;
  }
  for (int c = 0; c < nch; ++c) {
    const int64_t coff = static_cast<int64_t>(c) * (64 * D);
    f32x4 st[TPW][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      Frag<T> kf[KS], kl[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kf[s] = frag_load<T>(KC + coff + ktile_frag(kt, s, lane, D));
        if (kSplitKc<T>) kl[s] = frag_load<T>(KCL + coff + ktile_frag(kt, s, lane, D));
      }
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
        st[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          mma(st[qt][kt], kf[s], qf[qt][s]);
          if (kSplitKc<T>) mma(st[qt][kt], kl[s], qf[qt][s]);
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      float mx = kNegBig;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 64 * c + 16 * kt + 4 * grp + i;
          const float x = key < nvis[qt] ? st[qt][kt][i] * sl2 : -INFINITY;
          st[qt][kt][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = col_max4(mx);
      const float mn = fmaxf(m[qt], mx);
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += fast_exp2(st[qt][kt][i] - mn);
      ls[qt] = ls[qt] * fast_exp2(m[qt] - mn) + sum;
      m[qt] = mn;
    }
  }
  float lse2[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const float tot = col_sum4(ls[qt]);
    lse2[qt] = (nvis[qt] > 0 && colv) ? m[qt] + fast_log2(tot) : INFINITY;
  }

  // ---- pass 2: probabilities, compressed output, block scores
  const bool select = !a.inject;
  float* sc = reinterpret_cast<float*>(smem) + static_cast<size_t>(wave) * TPW * NcPad;
  f32x4 oacc[TPW][DT];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nch; ++c) {
    const int64_t coff = static_cast<int64_t>(c) * (64 * D);
    const S* vc = VC + coff;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f32x4 st[TPW][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        Frag<T> kf[KS], kl[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          kf[s] = frag_load<T>(KC + coff + ktile_frag(2 * s2 + h2, s, lane, D));
          if (kSplitKc<T>) kl[s] = frag_load<T>(KCL + coff + ktile_frag(2 * s2 + h2, s, lane, D));
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
            const int key = 64 * c + 32 * s2 + 16 * h2 + 4 * grp + i;
            st[qt][h2][i] = key < nvis[qt] ? fast_exp2(st[qt][h2][i] * sl2 - lse2[qt]) : 0.f;
          }
        if (select) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            f32x4 r;
            r.x = row_sum16(st[qt][h2].x);
            r.y = row_sum16(st[qt][h2].y);
            r.z = row_sum16(st[qt][h2].z);
            r.w = row_sum16(st[qt][h2].w);
            if (col == 0)
              *reinterpret_cast<f32x4*>(sc + qt * NcPad + 64 * c + 32 * s2 + 16 * h2 + 4 * grp) = r;
          }
        }
        const Frag<T> pf = pack_p<T>(st[qt][0], st[qt][1]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) mma(oacc[qt][dt], vf[dt], pf);
      }
    }
  }

  // ---- gate_cmp * O_cmp -> out (the other branches are added by k_sw)
  {
    const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0] + h * a.gs[2];
    SO* OUT = static_cast<SO*>(a.out) + b * a.os[0] + h * a.os[2] + 4 * grp;
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = t0 + qt;
      if (t < a.L && colv) {
        const float gc = to_f32<T>(GT[static_cast<int64_t>(t) * a.gs[1]]);
        SO* o = OUT + static_cast<int64_t>(t) * a.os[1];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4<O>(o + 16 * dt, oacc[qt][dt] * gc);
      }
    }
  }

  // ---- selection
  if (select) {
    wave_lds_sync();
    unsigned char* base = smem + static_cast<size_t>(nw) * TPW * NcPad * sizeof(float);
    uint64_t* surv = reinterpret_cast<uint64_t*>(base) + static_cast<size_t>(wave) * kSurvCap;
    int* selb = reinterpret_cast<int*>(base + static_cast<size_t>(nw) * kSurvCap * sizeof(uint64_t)) +
                wave * 64;
#pragma unroll 1
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = t0 + qt;
      if (t >= a.L) break;
      int32_t* row = a.idx + ((static_cast<int64_t>(b) * a.L + t) * a.G + g) * a.n;
      topk_wave(sc + qt * NcPad, t >> 6, a.n, row, surv, selb, lane);
    }
  }
}

// ------------------------------------------------------------------ k_sw

// One 32-key step of an online-softmax attention for one 16-column query
// tile: st holds the raw S^T of keys [kbase, kbase+32) in C layout; keys
// outside [klo, khi] are masked. Updates (m, l, acc) and returns nothing.
template <class T, int DT>
__device__ __forceinline__ void online_step(f32x4 (&st)[2], int kbase, int klo, int khi, int grp,
                                            float sl2, float& m, float& l, f32x4 (&acc)[DT],
                                            const Frag<T> (&vf)[DT]) {
  float mx = kNegBig;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kbase + 16 * h2 + 4 * grp + i;
      const float x = (key >= klo && key <= khi) ? st[h2][i] * sl2 : -INFINITY;
      st[h2][i] = x;
      mx = fmaxf(mx, x);
    }
  mx = col_max4(mx);
  const float mn = fmaxf(m, mx);
  const float alpha = fast_exp2(m - mn);
  float sum = 0.f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(st[h2][i] - mn);
      st[h2][i] = p;
      sum += p;
    }
  l = l * alpha + sum;
  m = mn;
  const Frag<T> pf = pack_p<T>(st[0], st[1]);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc[dt] *= alpha;
    mma(acc[dt], vf[dt], pf);
  }
}

template <class T, class O, int D, int TPW>
__global__ __launch_bounds__(256) void k_sw(PrefillArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int KS = D / 32, DT = D / 16;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int N = a.B * a.G * a.sw_tiles;
  const int per = (N + 7) >> 3;
  const int item = static_cast<int>(blockIdx.x & 7) * per + static_cast<int>(blockIdx.x >> 3);
  if (item >= N) return;
  const int g = item / (a.B * a.sw_tiles);
  const int rem = item % (a.B * a.sw_tiles);
  const int b = rem / a.sw_tiles, tile = rem % a.sw_tiles;
  const int t0 = (tile * nw + wave) * TPW;
  if (t0 >= a.L) return;
  const int col = lane & 15, grp = lane >> 4;
  const bool colv = col < a.Hg;
  const int h = g * a.Hg + col;
  const float sl2 = a.scale_log2;

  const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + h * a.qs[2] + 8 * grp;
  Frag<T> qf[TPW][KS];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = (t < a.L && colv) ? frag_load<T>(Q + static_cast<int64_t>(t) * a.qs[1] + 32 * s)
                                    : frag_zero<T>();
  }
  const int64_t tb = static_cast<int64_t>(b * a.G + g) * a.Nb * (64 * D);
  const S* KT = static_cast<const S*>(a.kt) + tb;
  const S* VT = static_cast<const S*>(a.vt) + tb;

  // ---- sliding window, shared by the wave's tokens
  const int tl = min(t0 + TPW - 1, a.L - 1);
  const int lo = max(0, t0 - a.w + 1);
  float mw[TPW], lw[TPW];
  f32x4 ow[TPW][DT];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    mw[qt] = kNegBig;
    lw[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ow[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int kb = lo & ~31; kb <= tl; kb += 32) {
    const int blk = kb >> 6, s2 = (kb >> 5) & 1;
    const S* kt = KT + static_cast<int64_t>(blk) * (64 * D);
    const S* vt = VT + static_cast<int64_t>(blk) * (64 * D);
    Frag<T> kf[2][KS];
    Frag<T> vf[DT];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[h2][s] = frag_load<T>(kt + ktile_frag(2 * s2 + h2, s, lane, D));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vt + vtile_frag(dt, s2, lane));
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = t0 + qt;
      f32x4 st[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        st[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(st[h2], kf[h2][s], qf[qt][s]);
      }
      // tokens past the end of the sequence see an empty range
      const int khi = t < a.L ? t : -1;
      online_step<T, DT>(st, kb, t - a.w + 1, khi, grp, sl2, mw[qt], lw[qt], ow[qt], vf);
    }
  }

  // ---- selected blocks, one token at a time, then the gate combination
  const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0] + h * a.gs[2];
  SO* OUT = static_cast<SO*>(a.out) + b * a.os[0] + h * a.os[2] + 4 * grp;
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    if (t >= a.L) break;
    const int own = t >> 6;
    const int32_t* row = a.idx + ((static_cast<int64_t>(b) * a.L + t) * a.G + g) * a.n;
    float ms = kNegBig, lsum = 0.f;
    f32x4 os[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) os[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int e = 0; e < a.n; ++e) {
      const int j = row[e];
      if (j < 0 || j > own) continue;
      const S* kt = KT + static_cast<int64_t>(j) * (64 * D);
      const S* vt = VT + static_cast<int64_t>(j) * (64 * D);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kb = 64 * j + 32 * s2;
        if (kb > t) break;
        Frag<T> kf[2][KS];
        Frag<T> vf[DT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int s = 0; s < KS; ++s) kf[h2][s] = frag_load<T>(kt + ktile_frag(2 * s2 + h2, s, lane, D));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vt + vtile_frag(dt, s2, lane));
        f32x4 st[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          st[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) mma(st[h2], kf[h2][s], qf[qt][s]);
        }
        online_step<T, DT>(st, kb, 0, t, grp, sl2, ms, lsum, os, vf);
      }
    }
    const float lst = col_sum4(lsum);
    const float lwt = col_sum4(lw[qt]);
    if (colv) {
      const int64_t gt = static_cast<int64_t>(t) * a.gs[1];
      const float gsl = to_f32<T>(GT[gt + 1]);
      const float gwn = to_f32<T>(GT[gt + 2]);
      const float fs = lst > 0.f ? gsl / lst : 0.f;
      const float fw = gwn / lwt;
      SO* o = OUT + static_cast<int64_t>(t) * a.os[1];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 prev = load4<O>(o + 16 * dt);
        store4<O>(o + 16 * dt, prev + os[dt] * fs + ow[qt][dt] * fw);
      }
    }
  }
}

// ------------------------------------------------------------------ launcher

static hipError_t record(hipEvent_t* ev, int i, hipStream_t st) {
  return ev != nullptr ? hipEventRecord(ev[i], st) : hipSuccess;
}

template <class T, class O, int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st, hipEvent_t* ev) {
  const size_t lds = a.inject ? 0 : cmp_lds_bytes(a.cmp_waves, a.NcT);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cmp<T, O, D, kCmpTPW>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int nblk_prep = max(a.Nb, a.NcT * 64);
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_prep<T, D>), dim3(nblk_prep, a.G, a.B), dim3(256), 0, st, a);
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_cmp<T, O, D, kCmpTPW>), dim3(a.B * a.G * a.cmp_tiles), dim3(64 * a.cmp_waves),
                     lds, st, a);
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
  const int N = a.B * a.G * a.sw_tiles;
  const int per = (N + 7) / 8;
  hipLaunchKernelGGL((k_sw<T, O, D, kSwTPW>), dim3(per * 8), dim3(64 * kSwWaves), 0, st, a);
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
