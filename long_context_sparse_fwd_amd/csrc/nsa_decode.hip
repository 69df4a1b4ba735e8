// NSA decode on gfx950: one new query token per sequence against a K/V cache
// and a block-mean cache, measured apart from prefill as the NSA how-to
// (qwbw.cn/news/106443), section 5, advises. The work is HBM-bound (each key
// is read once and used by the 16 heads of its group), so it is split into
// many 64-key chunks, one per wave, each producing a partial softmax state:
//
//  k_dec_scan     compressed chunks (64 blocks of the block cache) and window
//                 chunks (64 cache tokens); also stores the compressed logits.
//  k_dec_select   per (b, g): merge the compressed partials into the
//                 log-sum-exp and gate_cmp * O_cmp, form the block scores
//                 (probabilities summed over the group's heads) and select
//                 the own block + top-(n-1) earlier blocks (nsa_topk.h).
//  k_dec_sel      selected chunks: one selected 64-token block per wave.
//  k_dec_combine  merge window and selected partials, add the gated branches.
//
// K rows feed the S^T = K Q^T product straight from the cache; V rows go
// through LDS into the permuted V^T tile order the P.V product expects.
#include "nsa_device.h"
#include "nsa_internal.h"
#include "nsa_topk.h"

namespace nsa {

// floats per partial slot: m[16], l[16], O[16][D]
__host__ __device__ constexpr int dec_slot_floats(int D) { return 32 + 16 * D; }

__device__ __forceinline__ int dec_nslots(const DecodeArgs& a) { return 4 * (a.SC + a.SW + a.SS) + 1; }

__device__ __forceinline__ int dec_seqlen(const DecodeArgs& a, int b) {
  const int s = a.seqlens[b];
  return (s >= 1 && s <= a.Lmax) ? s : 0;  // 0 marks an invalid sequence
}

// One wave: attention of the group's 16 query columns over the keys
// [key0, key0 + 64) restricted to [klo, khi]; rows are read only inside that
// range. Writes the partial state (max, sum, unnormalised output) to `slot`
// and, if lrow != nullptr, the masked logits of the 64 keys to lrow[0..63].
template <class T, int D>
__device__ void dec_chunk(const typename T::storage* krows, int64_t kst,
                          const typename T::storage* vrows, int64_t vst, int key0, int klo,
                          int khi, const Frag<T> (&qf)[D / 32], float sl2,
                          typename T::storage* lv, float* slot, float* lrow, int lane) {
  using S = typename T::storage;
  constexpr int KS = D / 32, DT = D / 16;
  const int col = lane & 15, grp = lane >> 4;
  const int first = max(key0, klo), last = min(key0 + 63, khi);
  if (first > last) {
    if (grp == 0) {
      slot[col] = kNegBig;
      slot[16 + col] = 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(slot + 32 + col * D + 16 * dt + 4 * grp) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  f32x4 st[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = key0 + 16 * kt + col;
    const bool ok = key >= klo && key <= khi;
    Frag<T> kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[s] = ok ? frag_load<T>(krows + static_cast<int64_t>(key) * kst + 32 * s + 8 * grp)
                 : frag_zero<T>();
    st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) mma(st[kt], kf[s], qf[s]);
  }
  constexpr int VPR = D / 8;
  for (int e = lane; e < 64 * VPR; e += 64) {
    const int r = e / VPR, c = (e % VPR) * 8;
    const int key = key0 + r;
    __align__(16) S tmp[8];
    const Frag<T> vv = (key >= klo && key <= khi)
                           ? frag_load<T>(vrows + static_cast<int64_t>(key) * vst + c)
                           : frag_zero<T>();
    frag_store<T>(tmp, vv);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) lv[vtile_off(r, c + jj)] = tmp[jj];
  }
  wave_lds_sync();
  float mx = kNegBig;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 16 * kt + 4 * grp + i;
      const float x = (key >= klo && key <= khi) ? st[kt][i] * sl2 : -INFINITY;
      st[kt][i] = x;
      mx = fmaxf(mx, x);
    }
  if (lrow != nullptr) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) *reinterpret_cast<f32x4*>(lrow + 16 * kt + 4 * grp) = st[kt];
  }
  mx = col_max4(mx);
  float l = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(st[kt][i] - mx);
      st[kt][i] = p;
      l += p;
    }
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const Frag<T> pf = pack_p<T>(st[2 * s2], st[2 * s2 + 1]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) mma(o[dt], frag_load<T>(lv + vtile_frag(dt, s2, lane)), pf);
  }
  l = col_sum4(l);
  if (grp == 0) {
    slot[col] = mx;
    slot[16 + col] = l;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(slot + 32 + col * D + 16 * dt + 4 * grp) = o[dt];
  wave_lds_sync();
}

template <class T, int D>
__device__ __forceinline__ void dec_load_q(const DecodeArgs& a, int b, int g, int lane,
                                           Frag<T> (&qf)[D / 32]) {
  using S = typename T::storage;
  const int col = lane & 15, grp = lane >> 4;
  const bool ok = col < a.Hg;
  const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + (g * a.Hg + col) * a.qs[1] + 8 * grp;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) qf[s] = ok ? frag_load<T>(Q + 32 * s) : frag_zero<T>();
}

template <class T, int D>
__global__ __launch_bounds__(256) void k_dec_scan(DecodeArgs a) {
  using S = typename T::storage;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int sidx = blockIdx.y;
  const int seqlen = dec_seqlen(a, b);
  const int t = seqlen - 1;  // -1 for an invalid sequence: every chunk is empty
  S* lv = reinterpret_cast<S*>(smem) + wave * 64 * D;
  float* slot = a.part + (static_cast<int64_t>(bg) * dec_nslots(a)) * dec_slot_floats(D);
  Frag<T> qf[D / 32];
  dec_load_q<T, D>(a, b, g, lane, qf);
  if (sidx < a.SC) {
    const int key0 = (4 * sidx + wave) * 64;
    const int nvis = seqlen >> 6;
    const S* kr = static_cast<const S*>(a.kccache) + b * a.kcs[0] + g * a.kcs[1];
    const S* vr = static_cast<const S*>(a.vccache) + b * a.vcs[0] + g * a.vcs[1];
    float* lrow = a.logits + (static_cast<int64_t>(bg) * 16 + (lane & 15)) * a.NmaxPad + key0;
    dec_chunk<T, D>(kr, a.kcs[2], vr, a.vcs[2], key0, 0, nvis - 1, qf, a.scale_log2, lv,
                    slot + (4 * sidx + wave) * dec_slot_floats(D), lrow, lane);
  } else {
    const int ws = sidx - a.SC;
    const int wlo = max(0, seqlen - a.w);
    const int key0 = wlo + (4 * ws + wave) * 64;
    const S* kr = static_cast<const S*>(a.kcache) + b * a.ks[0] + g * a.ks[1];
    const S* vr = static_cast<const S*>(a.vcache) + b * a.vs[0] + g * a.vs[1];
    dec_chunk<T, D>(kr, a.ks[2], vr, a.vs[2], key0, wlo, t, qf, a.scale_log2, lv,
                    slot + (4 * a.SC + 4 * ws + wave) * dec_slot_floats(D), nullptr, lane);
  }
}

template <class T, int D>
__global__ __launch_bounds__(256) void k_dec_select(DecodeArgs a) {
  using S = typename T::storage;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sc = reinterpret_cast<float*>(smem);
  uint64_t* surv = reinterpret_cast<uint64_t*>(smem + a.NmaxPad * sizeof(float));
  int* selb = reinterpret_cast<int*>(surv + kSurvCap);
  float* Ms = reinterpret_cast<float*>(selb + 64);
  float* Ls = Ms + 16;
  float* L2 = Ls + 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int seqlen = dec_seqlen(a, b);
  constexpr int SF = dec_slot_floats(D);
  const float* P = a.part + static_cast<int64_t>(bg) * dec_nslots(a) * SF;
  float* cmp = a.part + (static_cast<int64_t>(bg) * dec_nslots(a) + dec_nslots(a) - 1) * SF + 32;
  int32_t* idxo = a.idx + static_cast<int64_t>(bg) * a.n;
  if (seqlen == 0) {
    if (!a.inject && tid < a.n) idxo[tid] = -1;
    for (int e = tid; e < 16 * D; e += 256) cmp[e] = 0.f;
    return;
  }
  const int t = seqlen - 1, nvis = seqlen >> 6, own = t >> 6;
  const int ncs = 4 * a.SC;
  if (tid < 16) {
    float M = kNegBig;
    for (int s = 0; s < ncs; ++s) M = fmaxf(M, P[s * SF + tid]);
    float L = 0.f;
    for (int s = 0; s < ncs; ++s) L += P[s * SF + 16 + tid] * fast_exp2(P[s * SF + tid] - M);
    Ms[tid] = M;
    Ls[tid] = L;
    L2[tid] = (nvis > 0 && tid < a.Hg) ? M + fast_log2(L) : INFINITY;
  }
  __syncthreads();
  const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0];
  for (int e = tid; e < 16 * D; e += 256) {
    const int hh = e / D, d = e % D;
    float acc = 0.f;
    for (int s = 0; s < ncs; ++s) acc += P[s * SF + 32 + e] * fast_exp2(P[s * SF + hh] - Ms[hh]);
    const float gc = hh < a.Hg ? to_f32<T>(GT[(g * a.Hg + hh) * a.gs[1]]) : 0.f;
    cmp[hh * D + d] = nvis > 0 ? acc / Ls[hh] * gc : 0.f;
  }
  if (a.inject) return;
  for (int j = tid; j < own; j += 256) {
    float s = 0.f;
    for (int hh = 0; hh < a.Hg; ++hh)
      s += fast_exp2(a.logits[(static_cast<int64_t>(bg) * 16 + hh) * a.NmaxPad + j] - L2[hh]);
    sc[j] = s;
  }
  __syncthreads();
  if (wave == 0) topk_wave(sc, own, a.n, idxo, surv, selb, lane);
}

template <class T, int D>
__global__ __launch_bounds__(256) void k_dec_sel(DecodeArgs a) {
  using S = typename T::storage;
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int e = 4 * blockIdx.y + wave;
  const int seqlen = dec_seqlen(a, b);
  const int t = seqlen - 1, own = t >> 6;
  S* lv = reinterpret_cast<S*>(smem) + wave * 64 * D;
  float* slot = a.part + (static_cast<int64_t>(bg) * dec_nslots(a) + 4 * (a.SC + a.SW) + e) *
                             dec_slot_floats(D);
  int j = -1;
  if (seqlen > 0 && e < a.n) j = a.idx[static_cast<int64_t>(bg) * a.n + e];
  const bool ok = j >= 0 && j <= own;
  Frag<T> qf[D / 32];
  dec_load_q<T, D>(a, b, g, lane, qf);
  const S* kr = static_cast<const S*>(a.kcache) + b * a.ks[0] + g * a.ks[1];
  const S* vr = static_cast<const S*>(a.vcache) + b * a.vs[0] + g * a.vs[1];
  // an unusable entry becomes an empty range (neutral partial)
  dec_chunk<T, D>(kr, a.ks[2], vr, a.vs[2], ok ? 64 * j : 0, 0, ok ? t : -1, qf, a.scale_log2, lv,
                  slot, nullptr, lane);
}

template <class T, class O, int D>
__global__ __launch_bounds__(256) void k_dec_combine(DecodeArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  __shared__ float Mw[16], Lw[16], Msl[16], Lsl[16];
  const int tid = threadIdx.x;
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int seqlen = dec_seqlen(a, b);
  constexpr int SF = dec_slot_floats(D);
  SO* OUT = static_cast<SO*>(a.out) + b * a.os[0];
  if (seqlen == 0) {
    for (int e = tid; e < a.Hg * D; e += 256)
      OUT[(g * a.Hg + e / D) * a.os[1] + e % D] = from_f32<O>(0.f);
    return;
  }
  const float* P = a.part + static_cast<int64_t>(bg) * dec_nslots(a) * SF;
  const float* W = P + 4 * a.SC * SF;
  const float* SL = P + 4 * (a.SC + a.SW) * SF;
  const float* cmp = P + (dec_nslots(a) - 1) * SF + 32;
  const int nw = 4 * a.SW, ns = 4 * a.SS;
  if (tid < 16) {
    float M = kNegBig, L = 0.f;
    for (int s = 0; s < nw; ++s) M = fmaxf(M, W[s * SF + tid]);
    for (int s = 0; s < nw; ++s) L += W[s * SF + 16 + tid] * fast_exp2(W[s * SF + tid] - M);
    Mw[tid] = M;
    Lw[tid] = L;
    M = kNegBig;
    L = 0.f;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, SL[s * SF + tid]);
    for (int s = 0; s < ns; ++s) L += SL[s * SF + 16 + tid] * fast_exp2(SL[s * SF + tid] - M);
    Msl[tid] = M;
    Lsl[tid] = L;
  }
  __syncthreads();
  const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0];
  for (int e = tid; e < a.Hg * D; e += 256) {
    const int hh = e / D, d = e % D;
    float ow = 0.f, osl = 0.f;
    for (int s = 0; s < nw; ++s) ow += W[s * SF + 32 + hh * D + d] * fast_exp2(W[s * SF + hh] - Mw[hh]);
    for (int s = 0; s < ns; ++s) osl += SL[s * SF + 32 + hh * D + d] * fast_exp2(SL[s * SF + hh] - Msl[hh]);
    const int h = g * a.Hg + hh;
    const float gsl = to_f32<T>(GT[h * a.gs[1] + 1]);
    const float gwn = to_f32<T>(GT[h * a.gs[1] + 2]);
    const float fs = Lsl[hh] > 0.f ? gsl / Lsl[hh] : 0.f;
    const float v = cmp[hh * D + d] + osl * fs + ow * (gwn / Lw[hh]);
    OUT[h * a.os[1] + d] = from_f32<O>(v);
  }
}

static hipError_t record(hipEvent_t* ev, int i, hipStream_t st) {
  return ev != nullptr ? hipEventRecord(ev[i], st) : hipSuccess;
}

template <class T, class O, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st, hipEvent_t* ev) {
  using S = typename T::storage;
  const size_t lds_chunk = 4 * 64 * D * sizeof(S);
  const size_t lds_sel = a.NmaxPad * sizeof(float) + kSurvCap * sizeof(uint64_t) + 64 * sizeof(int) +
                         48 * sizeof(float);
  hipError_t e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_scan<T, D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_chunk));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_sel<T, D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_chunk));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_select<T, D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_sel));
  if (e != hipSuccess) return e;
  const int BG = a.B * a.G;
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_scan<T, D>), dim3(BG, a.SC + a.SW), dim3(256), lds_chunk, st, a);
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_select<T, D>), dim3(BG), dim3(256), lds_sel, st, a);
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_sel<T, D>), dim3(BG, a.SS), dim3(256), lds_chunk, st, a);
  if ((e = record(ev, 3, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_combine<T, O, D>), dim3(BG), dim3(256), 0, st, a);
  if ((e = record(ev, 4, st)) != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool in_bf16, bool out_bf16, hipStream_t st,
                         hipEvent_t* ev) {
  if (in_bf16) {
    if (out_bf16)
      return a.D == 64 ? launch_decode_t<BF16, BF16, 64>(a, st, ev)
                       : launch_decode_t<BF16, BF16, 128>(a, st, ev);
    return a.D == 64 ? launch_decode_t<BF16, F32, 64>(a, st, ev)
                     : launch_decode_t<BF16, F32, 128>(a, st, ev);
  }
  return a.D == 64 ? launch_decode_t<F32, F32, 64>(a, st, ev) : launch_decode_t<F32, F32, 128>(a, st, ev);
}

}  // namespace nsa
