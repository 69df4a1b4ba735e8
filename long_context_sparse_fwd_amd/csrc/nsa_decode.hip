// NSA decode on gfx950: one new query token per sequence against a K/V cache
// and a block-mean cache, measured apart from prefill as the NSA how-to
// (qwbw.cn/news/106443), section 5, advises. The work is HBM-bound: every key
// is read once and serves the 16 query heads of its group, so the kernels
// are organised around keeping many 32 KiB chunks in flight.
//
//  k_dec_scan    grid (sequence x group, compressed splits + window splits).
//                Each wave loads one 64-key chunk (64 block means, or 64
//                window tokens) into registers, attends the group's 16 heads
//                over it, and the workgroup merges its 4 waves into one
//                partial softmax state (max, sum, unnormalised output). The
//                compressed splits also store their logits for the scores.
//  k_dec_finish  one workgroup per (sequence, group): merges the compressed
//                partials into the log-sum-exp and gate_cmp * O_cmp, forms
//                the block scores (probabilities summed over the group's
//                heads), selects the own block + top-(n-1) earlier blocks
//                (nsa_topk.h), gathers the selected blocks across its waves,
//                and adds the gated selected and window branches into out.
//
// K rows feed the S^T = K Q^T product straight from the cache; V rows go
// through LDS into the permuted V^T tile order of the P.V product.
#include "nsa_device.h"
#include "nsa_internal.h"
#include "nsa_topk.h"

namespace nsa {

// floats per partial slot: m[16], l[16], O[16][D]
__host__ __device__ constexpr int dec_slot_floats(int D) { return 32 + 16 * D; }

__device__ __forceinline__ int dec_seqlen(const DecodeArgs& a, int b) {
  const int s = a.seqlens[b];
  return (s >= 1 && s <= a.Lmax) ? s : 0;  // 0 marks an invalid sequence
}

// One wave's registers for a 64-key chunk: the K rows as A operands and the V
// rows as 8-element vectors (lane l holds rows l/(D/8) + 64 i/(D/8)).
template <class T, int D>
struct Chunk {
  Frag<T> k[4][D / 32];
  Frag<T> v[D / 8];
};

// Loads keys [key0, key0 + 64) restricted to [klo, khi]; rows outside are
// zero and never read.
template <class T, int D>
__device__ __forceinline__ void chunk_load(Chunk<T, D>& c, const typename T::storage* krows,
                                           int64_t kst, const typename T::storage* vrows,
                                           int64_t vst, int key0, int klo, int khi, int lane) {
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = key0 + 16 * kt + col;
    const bool ok = key >= klo && key <= khi;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      c.k[kt][s] = ok ? frag_load<T>(krows + static_cast<int64_t>(key) * kst + 32 * s + 8 * grp)
                      : frag_zero<T>();
  }
  constexpr int VPR = D / 8;
#pragma unroll
  for (int i = 0; i < VPR; ++i) {
    const int e = lane + 64 * i;
    const int key = key0 + e / VPR;
    const bool ok = key >= klo && key <= khi;
    c.v[i] = ok ? frag_load<T>(vrows + static_cast<int64_t>(key) * vst + (e % VPR) * 8) : frag_zero<T>();
  }
}

// Online-softmax update of (m, l, acc) with one loaded chunk. lv: this wave's
// 64*D elements of LDS. lrow (optional): receives the masked log2-domain
// logits of the chunk's 64 keys for this lane's query column.
template <class T, int D>
__device__ __forceinline__ void chunk_attend(const Chunk<T, D>& c, int key0, int klo, int khi,
                                             const Frag<T> (&qf)[D / 32], float sl2,
                                             typename T::storage* lv, float& m, float& l,
                                             f32x4 (&acc)[D / 16], float* lrow, int lane) {
  using S = typename T::storage;
  constexpr int KS = D / 32, DT = D / 16, VPR = D / 8;
  const int grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < VPR; ++i) {
    const int e = lane + 64 * i;
    const int r = e / VPR, cc = (e % VPR) * 8;
    __align__(16) S tmp[8];
    frag_store<T>(tmp, c.v[i]);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) lv[vtile_off(r, cc + jj)] = tmp[jj];
  }
  f32x4 st[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) mma(st[kt], c.k[kt][s], qf[s]);
  }
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
  const float mn = fmaxf(m, mx);
  const float alpha = fast_exp2(m - mn);
  float sum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(st[kt][i] - mn);
      st[kt][i] = p;
      sum += p;
    }
  l = l * alpha + sum;
  m = mn;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
  wave_lds_sync();
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const Frag<T> pf = pack_p<T>(st[2 * s2], st[2 * s2 + 1]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) mma(acc[dt], frag_load<T>(lv + vtile_frag(dt, s2, lane)), pf);
  }
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

// Stores a wave's partial state (m per column, l summed over the column's
// lanes, O^T accumulators) as m[16], l[16], O[16][D] at dst.
template <int D>
__device__ __forceinline__ void store_partial(float* dst, float m, float l, const f32x4 (&acc)[D / 16],
                                              int lane) {
  const int col = lane & 15, grp = lane >> 4;
  if (grp == 0) {
    dst[col] = m;
    dst[16 + col] = l;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4*>(dst + 32 + col * D + 16 * dt + 4 * grp) = acc[dt];
}

// Merges `cnt` partial slots (stride SF floats) for head h: returns the
// merged (max, sum); the output merge is done element-wise by the caller.
__device__ __forceinline__ void merge_stats(const float* p, int cnt, int SF, int h, float& M, float& L) {
  M = kNegBig;
  for (int s = 0; s < cnt; ++s) M = fmaxf(M, p[s * SF + h]);
  L = 0.f;
  for (int s = 0; s < cnt; ++s) L += p[s * SF + 16 + h] * fast_exp2(p[s * SF + h] - M);
}

template <class T, int D>
__global__ __launch_bounds__(256) void k_dec_scan(DecodeArgs a) {
  using S = typename T::storage;
  constexpr int SF = dec_slot_floats(D), DT = D / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int sidx = blockIdx.y;
  const int seqlen = dec_seqlen(a, b);
  const int t = seqlen - 1;  // -1 for an invalid sequence: every chunk is empty
  S* lv = reinterpret_cast<S*>(smem) + wave * 64 * D;
  Frag<T> qf[D / 32];
  dec_load_q<T, D>(a, b, g, lane, qf);

  int key0, klo, khi;
  const S *kr, *vr;
  int64_t kst, vst;
  float* lrow = nullptr;
  if (sidx < a.SC) {
    key0 = (4 * sidx + wave) * 64;
    klo = 0;
    khi = (seqlen >> 6) - 1;
    kr = static_cast<const S*>(a.kccache) + b * a.kcs[0] + g * a.kcs[1];
    vr = static_cast<const S*>(a.vccache) + b * a.vcs[0] + g * a.vcs[1];
    kst = a.kcs[2];
    vst = a.vcs[2];
    lrow = a.logits + (static_cast<int64_t>(bg) * 16 + (lane & 15)) * a.NmaxPad + key0;
  } else {
    const int wlo = max(0, seqlen - a.w);
    key0 = wlo + (4 * (sidx - a.SC) + wave) * 64;
    klo = wlo;
    khi = t;
    kr = static_cast<const S*>(a.kcache) + b * a.ks[0] + g * a.ks[1];
    vr = static_cast<const S*>(a.vcache) + b * a.vs[0] + g * a.vs[1];
    kst = a.ks[2];
    vst = a.vs[2];
  }
  float m = kNegBig, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (max(key0, klo) <= min(key0 + 63, khi)) {
    Chunk<T, D> c;
    chunk_load<T, D>(c, kr, kst, vr, vst, key0, klo, khi, lane);
    chunk_attend<T, D>(c, key0, klo, khi, qf, a.scale_log2, lv, m, l, acc, lrow, lane);
  }
  l = col_sum4(l);
  // merge the 4 waves through LDS (reusing the V staging area)
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(smem);
  store_partial<D>(mrg + wave * SF, m, l, acc, lane);
  __syncthreads();
  float* slot = a.part + (static_cast<int64_t>(bg) * (a.SC + a.SW) + sidx) * SF;
  if (tid < 16) {
    float M, L;
    merge_stats(mrg, 4, SF, tid, M, L);
    slot[tid] = M;
    slot[16 + tid] = L;
  }
  for (int e = tid; e < 16 * D; e += 256) {
    const int h = e / D;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg[w * SF + h]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o += mrg[w * SF + 32 + e] * fast_exp2(mrg[w * SF + h] - M);
    slot[32 + e] = o;
  }
}

template <class T, class O, int D, int FW>
__global__ __launch_bounds__(512) void k_dec_finish(DecodeArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int SF = dec_slot_floats(D), DT = D / 16, NT = 64 * FW;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sc = reinterpret_cast<float*>(smem);
  uint64_t* surv = reinterpret_cast<uint64_t*>(sc + a.NmaxPad);
  int* selb = reinterpret_cast<int*>(surv + kSurvCap);
  int* selo = selb + 64;
  float* hs = reinterpret_cast<float*>(selo + 64);  // per head: M, L, lse2, g_cmp
  float* ocmp = hs + 64;                            // [16][D]
  unsigned char* big = reinterpret_cast<unsigned char*>(ocmp + 16 * D);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int seqlen = dec_seqlen(a, b);
  const int nslot = a.SC + a.SW;
  const float* P = a.part + static_cast<int64_t>(bg) * nslot * SF;
  int32_t* idxo = a.idx + static_cast<int64_t>(bg) * a.n;
  const S* GT = static_cast<const S*>(a.gates) + b * a.gs[0];
  SO* OUT = static_cast<SO*>(a.out) + b * a.os[0];
  if (seqlen == 0) {
    for (int e = tid; e < a.Hg * D; e += NT) OUT[(g * a.Hg + e / D) * a.os[1] + e % D] = from_f32<O>(0.f);
    if (!a.inject && tid < a.n) idxo[tid] = -1;
    return;
  }
  const int t = seqlen - 1, nvis = seqlen >> 6, own = t >> 6;

  // ---- compressed branch: merge the partials, log-sum-exp, gated output
  if (tid < 16) {
    float M, L;
    merge_stats(P, a.SC, SF, tid, M, L);
    hs[4 * tid] = M;
    hs[4 * tid + 1] = L;
    hs[4 * tid + 2] = (nvis > 0 && tid < a.Hg) ? M + fast_log2(L) : INFINITY;
    hs[4 * tid + 3] = tid < a.Hg ? to_f32<T>(GT[(g * a.Hg + tid) * a.gs[1]]) : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < 16 * D; e += NT) {
    const int h = e / D;
    float o = 0.f;
    for (int s = 0; s < a.SC; ++s) o += P[s * SF + 32 + e] * fast_exp2(P[s * SF + h] - hs[4 * h]);
    ocmp[e] = nvis > 0 ? o / hs[4 * h + 1] * hs[4 * h + 3] : 0.f;
  }

  // ---- block scores and selection
  if (!a.inject) {
    for (int j = tid; j < own; j += NT) {
      float s = 0.f;
      for (int h = 0; h < a.Hg; ++h)
        s += fast_exp2(a.logits[(static_cast<int64_t>(bg) * 16 + h) * a.NmaxPad + j] - hs[4 * h + 2]);
      sc[j] = s;
    }
    __syncthreads();
    if (wave == 0) topk_wave(sc, own, a.n, selo, surv, selb, lane);
    __syncthreads();
    if (tid < a.n) idxo[tid] = selo[tid];
  } else {
    if (tid < a.n) selo[tid] = idxo[tid];
    __syncthreads();
  }

  // ---- selected blocks, spread over the waves
  Frag<T> qf[D / 32];
  dec_load_q<T, D>(a, b, g, lane, qf);
  const S* kr = static_cast<const S*>(a.kcache) + b * a.ks[0] + g * a.ks[1];
  const S* vr = static_cast<const S*>(a.vcache) + b * a.vs[0] + g * a.vs[1];
  S* lv = reinterpret_cast<S*>(big) + wave * 64 * D;
  float m = kNegBig, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int e = wave; e < a.n; e += FW) {
    const int j = selo[e];
    if (j < 0 || j > own) continue;  // unusable injected entry
    Chunk<T, D> c;
    chunk_load<T, D>(c, kr, a.ks[2], vr, a.vs[2], 64 * j, 64 * j, t, lane);
    chunk_attend<T, D>(c, 64 * j, 64 * j, t, qf, a.scale_log2, lv, m, l, acc, nullptr, lane);
  }
  l = col_sum4(l);
  __syncthreads();
  float* wp = reinterpret_cast<float*>(big);  // per-wave partials, reusing the V staging
  store_partial<D>(wp + wave * SF, m, l, acc, lane);
  __syncthreads();

  // ---- merge selected (in LDS) and window (from k_dec_scan) partials, combine
  const float* W = P + a.SC * SF;
  if (tid < 16) {  // per head: max and gate-scaled reciprocal sum of each branch
    float Ms, Ls, Mw, Lw;
    merge_stats(wp, FW, SF, tid, Ms, Ls);
    merge_stats(W, a.SW, SF, tid, Mw, Lw);
    const int hq = g * a.Hg + tid;
    const float gsl = tid < a.Hg ? to_f32<T>(GT[hq * a.gs[1] + 1]) : 0.f;
    const float gwn = tid < a.Hg ? to_f32<T>(GT[hq * a.gs[1] + 2]) : 0.f;
    hs[4 * tid] = Ms;
    hs[4 * tid + 1] = Ls > 0.f ? gsl / Ls : 0.f;
    hs[4 * tid + 2] = Mw;
    hs[4 * tid + 3] = Lw > 0.f ? gwn / Lw : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < a.Hg * D; e += NT) {
    const int h = e / D;
    float os = 0.f, ow = 0.f;
#pragma unroll
    for (int w = 0; w < FW; ++w) os += wp[w * SF + 32 + e] * fast_exp2(wp[w * SF + h] - hs[4 * h]);
    for (int s = 0; s < a.SW; ++s) ow += W[s * SF + 32 + e] * fast_exp2(W[s * SF + h] - hs[4 * h + 2]);
    const float v = ocmp[e] + os * hs[4 * h + 1] + ow * hs[4 * h + 3];
    OUT[(g * a.Hg + h) * a.os[1] + e % D] = from_f32<O>(v);
  }
}

size_t dec_finish_lds_bytes(int NmaxPad, int D, bool bf16) {
  const int FW = bf16 ? 8 : 4;
  const size_t el = bf16 ? 2 : 4;
  const size_t stage = static_cast<size_t>(FW) * 64 * D * el;
  const size_t parts = static_cast<size_t>(FW) * dec_slot_floats(D) * sizeof(float);
  return NmaxPad * sizeof(float) + kSurvCap * sizeof(uint64_t) + 128 * sizeof(int) +
         64 * sizeof(float) + 16 * D * sizeof(float) + (stage > parts ? stage : parts);
}

size_t dec_scan_lds_bytes(int D, bool bf16) {
  const size_t stage = 4 * 64 * static_cast<size_t>(D) * (bf16 ? 2 : 4);
  const size_t parts = 4 * static_cast<size_t>(dec_slot_floats(D)) * sizeof(float);
  return stage > parts ? stage : parts;
}

static hipError_t record(hipEvent_t* ev, int i, hipStream_t st) {
  return ev != nullptr ? hipEventRecord(ev[i], st) : hipSuccess;
}

template <class T, class O, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st, hipEvent_t* ev) {
  constexpr bool kBf16 = sizeof(typename T::storage) == 2;
  constexpr int FW = kBf16 ? 8 : 4;
  const size_t lds_scan = dec_scan_lds_bytes(D, kBf16);
  const size_t lds_fin = dec_finish_lds_bytes(a.NmaxPad, D, kBf16);
  hipError_t e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_scan<T, D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_scan));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_finish<T, O, D, FW>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_fin));
  if (e != hipSuccess) return e;
  const int BG = a.B * a.G;
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_scan<T, D>), dim3(BG, a.SC + a.SW), dim3(256), lds_scan, st, a);
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_dec_finish<T, O, D, FW>), dim3(BG), dim3(64 * FW), lds_fin, st, a);
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
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
