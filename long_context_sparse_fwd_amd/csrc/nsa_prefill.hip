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
#include <algorithm>
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
// plus a bf16 low part (hi + lo holds ~16 significant bits), and the
// compressed-branch QK products of the scoring pass add the low part with a
// second MFMA where it matters (kLoMinBlocks).
template <class T>
constexpr bool kSplitKc = false;
template <>
constexpr bool kSplitKc<BF16> = true;

// Queries that see at least this many block means score them from the high
// parts alone (plain geometry). A block score is a head sum of probabilities
// of about 1/n each among n visible blocks, so the relative logit error of
// the bf16 high part (~2^-9 per element) moves a score by O(1/n): measured
// over random i.i.d. N(0,1) rows at 512 blocks, at most 7.6e-6 (median
// 5.5e-6), against 1e-4 gaps the selection has to resolve exactly; at 64
// blocks the same error reaches 6.9e-5, hence the low parts below the bound.
constexpr int kLoMinBlocks = 512;

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

// Compressed blocks visible to query t: those whose last token i*cd + cl - 1
// is at or before t.
__device__ __forceinline__ int nvis_of(const PrefillArgs& a, int t) {
  return t + 1 >= a.cl ? (t + 1 - a.cl) / a.cd + 1 : 0;
}

// Gate c (compressed, selected, window) of query row `row` and head h: the
// gate layer's fp32 output when there is one, else the given gates.
template <class T>
__device__ __forceinline__ float gate_of(const PrefillArgs& a, int b, int row, int h, int c) {
  if (a.gates32 != nullptr) return a.gates32[((static_cast<int64_t>(b) * a.Lq + row) * a.Hq + h) * 3 + c];
  const typename T::storage* GT = static_cast<const typename T::storage*>(a.gates);
  return to_f32<T>(GT[b * a.gs[0] + static_cast<int64_t>(row) * a.gs[1] + h * a.gs[2] + c]);
}

// Gate components c[0..NC) of query rows row[0..N) of head h, all read
// before any is used (one wait, not one per read): the branch on where the
// gates live sits outside the reads.
template <class T, int N, int NC>
__device__ __forceinline__ void gates_of(const PrefillArgs& a, int b, const int (&row)[N], int h, const int (&c)[NC],
                                         float (&g)[N][NC]) {
  if (a.gates32 != nullptr) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < NC; ++j) g[i][j] = a.gates32[((static_cast<int64_t>(b) * a.Lq + row[i]) * a.Hq + h) * 3 + c[j]];
  } else {
    const typename T::storage* GT = static_cast<const typename T::storage*>(a.gates);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < NC; ++j)
        g[i][j] = to_f32<T>(GT[b * a.gs[0] + static_cast<int64_t>(row[i]) * a.gs[1] + h * a.gs[2] + c[j]]);
  }
}

// Element j (0..7) of a fragment.
template <class T>
__device__ __forceinline__ float frag_elem(const Frag<T>& f, int j);
template <>
__device__ __forceinline__ float frag_elem<BF16>(const Frag<BF16>& f, int j) {
  const uint32_t w = f.v[j >> 1];
  return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float frag_elem<F32>(const Frag<F32>& f, int j) {
  return j < 4 ? f.lo[j] : f.hi[j - 4];
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
  if (a.cmp_in_prep && j < a.NcT * 64) {
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
      sk *= a.scale_log2;  // K means are kept as log2-domain logit factors
      const S hi = from_f32<T>(sk);
      kc[ktile_off(r, d, D)] = hi;
      if (kSplitKc<T>) kcl[ktile_off(r, d, D)] = from_f32<T>(sk - to_f32<T>(hi));
      vc[vtile_off(r, d)] = from_f32<T>(sv);
    }
  }
}

// ------------------------------------------------------------------ k_ctile

// Compressed tiles for the general geometry: compressed block i of (b, g)
// summarises tokens [i*cd, i*cd + cl) -- their mean, or the learned linear map
// w[o][p][c] of the flattened block plus bias[o] (each block compressed into
// one representation by a learned projection: NSA factory write-up,
// chencunli.com, section "What dynamic sparsity actually sparsifies").
// Workgroup (x, g, b): 64 compressed blocks, of K for even x and of V for odd
// x. The learned map is a [64 x cl*D] by [cl*D x D] product on MFMA: wave w
// takes rows 16w..16w+15 and all D outputs, the reduction running over
// (position, input dim) in steps of 32. Rows past Nc are written as zeros.
template <class T, int D>
__global__ __launch_bounds__(256) void k_ctile(PrefillArgs a) {
  using S = typename T::storage;
  const int c = blockIdx.x >> 1, is_v = blockIdx.x & 1, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Lb = __builtin_amdgcn_readfirstlane(seq_span(a, b).L);  // key rows past it read as zero
  const S* X = static_cast<const S*>(is_v ? a.v : a.k) + b * (is_v ? a.vs[0] : a.ks[0]) +
               g * (is_v ? a.vs[2] : a.ks[2]);
  const int64_t xs = is_v ? a.vs[1] : a.ks[1];
  const int64_t tile = (static_cast<int64_t>(b * a.G + g) * a.NcT + c) * (64 * D);
  S* hi_t = static_cast<S*>(is_v ? a.vct : a.kct) + tile;
  S* lo_t = (kSplitKc<T> && !is_v) ? static_cast<S*>(a.kclt) + tile : nullptr;
  auto put = [&](int r, int d, float x) {
    if (is_v) {
      hi_t[vtile_off(r, d)] = from_f32<T>(x);
    } else {
      x *= a.scale_log2;  // K representations are kept as log2-domain logit factors
      const S h = from_f32<T>(x);
      hi_t[ktile_off(r, d, D)] = h;
      if (kSplitKc<T>) lo_t[ktile_off(r, d, D)] = from_f32<T>(x - to_f32<T>(h));
    }
  };
  const void* wp = is_v ? a.wv : a.wk;
  if (wp == nullptr) {
    for (int e = tid; e < 64 * D; e += 256) {
      const int r = e / D, d = e % D, i = 64 * c + r;
      float sum = 0.f;
      if (i < a.Nc) {
        const int t0 = i * a.cd, t1 = min(t0 + a.cl, Lb);
        for (int t = t0; t < t1; ++t) sum += to_f32<T>(X[static_cast<int64_t>(t) * xs + d]);
        sum *= a.inv_cl;
      }
      put(r, d, sum);
    }
    return;
  }
  const S* W = static_cast<const S*>(wp);
  const S* bias = static_cast<const S*>(is_v ? a.bv : a.bk);
  constexpr int DT = D / 16, KS = D / 32;
  const int i = 64 * c + 16 * wave + (lane & 15);  // this lane's row of the A operand
  const bool row_ok = i < a.Nc;
  const int t0 = i * a.cd;
  f32x4 acc[DT];
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.cl; ++p) {
    const int t = t0 + p;
    const bool tok = row_ok && t < Lb;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * ks + 8 * (lane >> 4);
      const Frag<T> af = tok ? frag_load<T>(X + static_cast<int64_t>(t) * xs + c0) : frag_zero<T>();
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        const int o = 16 * nt + (lane & 15);
        mma(acc[nt], af, frag_load<T>(W + (static_cast<int64_t>(o) * a.cl + p) * D + c0));
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
    const int o = 16 * nt + (lane & 15);
    const float bo = to_f32<T>(bias[o]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 16 * wave + 4 * (lane >> 4) + k;
      put(r, o, 64 * c + r < a.Nc ? acc[nt][k] + bo : 0.f);
    }
  }
}

// ------------------------------------------------------------------ k_gate

// Gate layer: gates32[b][row][h][c] = sigmoid(q[b][row][h] . gate_w[h][:, c] +
// gate_b[h][c]) in fp32, one thread per (b, row, head). The gates of the
// three branches are learned (NSA how-to, qwbw.cn/news/106443, section 3,
// gate_type learned); here a one-layer map of the head's query.
template <class T, int D>
__global__ __launch_bounds__(256) void k_gate(PrefillArgs a) {
  using S = typename T::storage;
  const S* W = static_cast<const S*>(a.gate_w);
  const S* Bg = static_cast<const S*>(a.gate_b);
  const int64_t n = static_cast<int64_t>(a.B) * a.Lq * a.Hq;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(256) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int h = static_cast<int>(e % a.Hq);
    const int64_t br = e / a.Hq;
    const int row = static_cast<int>(br % a.Lq), b = static_cast<int>(br / a.Lq);
    const S* q = static_cast<const S*>(a.q) + b * a.qs[0] + static_cast<int64_t>(row) * a.qs[1] + h * a.qs[2];
    const S* w = W + static_cast<int64_t>(h) * D * 3;
    float z0 = to_f32<T>(Bg[3 * h]), z1 = to_f32<T>(Bg[3 * h + 1]), z2 = to_f32<T>(Bg[3 * h + 2]);
    for (int d0 = 0; d0 < D; d0 += 8) {
      const Frag<T> f = frag_load<T>(q + d0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = frag_elem<T>(f, j);
        const S* wr = w + 3 * (d0 + j);
        z0 = fmaf(x, to_f32<T>(wr[0]), z0);
        z1 = fmaf(x, to_f32<T>(wr[1]), z1);
        z2 = fmaf(x, to_f32<T>(wr[2]), z2);
      }
    }
    float* o = a.gates32 + e * 3;
    o[0] = 1.0f / (1.0f + fast_exp2(-z0 * kLog2e));
    o[1] = 1.0f / (1.0f + fast_exp2(-z1 * kLog2e));
    o[2] = 1.0f / (1.0f + fast_exp2(-z2 * kLog2e));
  }
}

// Selection-block scores from the compressed-block scores of one token, in
// place (sc[0 .. own) on return): the compressed-attention mass on each
// selection block's tokens, every compressed block's probability spread evenly
// over its cl tokens. Selection block j reads compressed blocks i >= j only
// (cl <= ls, cd <= cl), so rounds of 64 blocks can overwrite the scores they
// have consumed. Whole wave, uniform arguments.
__device__ inline void map_selection_scores(const PrefillArgs& a, float* sc, int own, int nv, int lane) {
  for (int r0 = 0; r0 < own; r0 += 64) {
    const int j = r0 + lane;
    float sum = 0.f;
    if (j < own) {
      const int lo = j * a.ls, hi = lo + a.ls;
      const int x = lo - a.cl + 1;
      const int i0 = x <= 0 ? 0 : (x + a.cd - 1) / a.cd;
      const int i1 = min(nv - 1, (hi - 1) / a.cd);
      for (int i = i0; i <= i1; ++i) {
        const int blo = i * a.cd;
        sum = fmaf(sc[i], static_cast<float>(min(blo + a.cl, hi) - max(blo, lo)), sum);
      }
      sum *= a.inv_cl;
    }
    wave_lds_sync();
    if (j < own) sc[j] = sum;
    wave_lds_sync();
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

template <class T, class O, int D, int NW, bool LOL, bool GSC>
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
  Frag<T> qf[TPW][KS];
  float gcmp[TPW], gwin[TPW];
  int nvis[TPW];
  // reads at clamped (token, head) indices, zeroed where not valid
  const S* Qc = static_cast<const S*>(a.q) + b * a.qs[0] + (colv ? h : g * a.Hg) * a.qs[2] + 8 * grp;
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = tw + qt, tc = min(t, Le - 1);
    const bool valid = t < Le && colv;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = frag_load_if<T>(Qc + static_cast<int64_t>(tc - t0q) * a.qs[1] + 32 * s, valid);
  }
  {
    int rows[TPW];
    float gv[TPW][2];
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) rows[qt] = min(tw + qt, Le - 1) - t0q;
    gates_of<T>(a, b, rows, colv ? h : g * a.Hg, {0, 2}, gv);
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = tw + qt;
      const bool valid = t < Le && colv;
      gcmp[qt] = valid ? gv[qt][0] : 0.f;
      gwin[qt] = valid ? gv[qt][1] : 0.f;
      nvis[qt] = t < Le ? nvis_of(a, t) : 0;
    }
  }
  f32x4 oacc[TPW][DT];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  TileStager<T, D, NT> stg;

  // The three phases below (window, compressed pass 1, compressed pass 2)
  // step over 64-key chunks x = 0 .. n-1 in two segments each, separated by
  // LDS barriers: segment 1 is the softmax arithmetic of chunk x (VALU),
  // segment 2 the P.V products of chunk x and the Q.K products of chunk
  // x + 1 (MFMA). Waves w and w + 4 share a SIMD; waves 4..7 run one segment
  // behind waves 0..3, so between two barriers one wave of every SIMD does
  // vector work while the other keeps the matrix unit busy.
  // Staging: stage buffer y & 1 holds K (and the low part of K) and V of
  // chunk y. D(y) = {K(y), V(y - 1)} (indices clamped to the last chunk)
  // replaces K(y - 2) and V(y - 3); each wave loads and stores its share of
  // D(y) within one segment 1 (so the loaded registers are not live across
  // the products): the trailing waves in segment 1 of chunk y - 2, the
  // leading ones in segment 1 of chunk y - 1, one period later. Both periods
  // come after the last reads of K(y - 2) and V(y - 3) (the trailing waves'
  // segment 2 of chunk y - 3) and before the first read of D(y) (the leading
  // waves' segment 2 of chunk y - 1), and in neither does the other group
  // read the slots being written.
  const bool trail = NW == 8 && wave >= 4;
  // Masks compare the lane's key offset g4 = 4 grp with wave-uniform bounds,
  // so no per-key lane offsets stay live.
  const int g4 = 4 * grp;

  static_assert(TPW == 2, "the low-part products below are written for two tokens per wave");
  // S^T of one 64-key chunk for the wave's tokens, accumulated onto init[qt]:
  // st[qt][kt][i] holds key 16 kt + 4 grp + i of the chunk, head col. Token
  // qt adds the products with the low parts kl when lo[qt] (wave-uniform).
  // The k-steps are the outer loop: the eight accumulators (4 key tiles x 2
  // tokens) each take one product per k-step, so consecutive products do not
  // depend on each other (an MFMA that accumulates onto the previous one's
  // result waits for it to finish).
  auto qk_chunk = [&](const S* kb, const S* kl, const bool (&lo)[TPW], const f32x4 (&init)[TPW],
                      f32x4 (&st)[TPW][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) st[qt][kt] = init[qt];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      Frag<T> kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[kt] = frag_load<T>(kb + ktile_frag(kt, s, lane, D));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < TPW; ++qt) mma(st[qt][kt], kf[kt], qf[qt][s]);
    }
    if (kSplitKc<T> && lo[0]) {  // the low parts after the high ones (lo[1] implies lo[0])
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag<T> kf[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kf[kt] = frag_load<T>(kl + ktile_frag(kt, s, lane, D));
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mma(st[0][kt], kf[kt], qf[0][s]);
        if (lo[1]) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) mma(st[1][kt], kf[kt], qf[1][s]);
        }
      }
    }
  };
  // acc[qt] += V^T . P^T over one 64-key chunk; pf[qt][s2] holds the
  // probabilities of keys [32 s2, 32 s2 + 32) (pack_p order). With lacc, the
  // softmax denominators too, on the matrix unit: a product with an all-ones
  // A operand sums the packed probabilities over the keys, and every lane of
  // a column receives its head's sum (the two products of an accumulator
  // are sixteen products apart).
  const Frag<T> ones = frag_ones<T>();
  auto pv_chunk = [&](const S* vb, const Frag<T> (&pf)[TPW][2], f32x4 (*lacc)[TPW]) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      Frag<T> vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vb + vtile_frag(dt, s2, lane));
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) mma(oacc[qt][dt], vf[dt], pf[qt][s2]);
      if (lacc != nullptr) {
#pragma unroll
        for (int qt = 0; qt < TPW; ++qt) mma((*lacc)[qt], ones, pf[qt][s2]);
      }
    }
  };
  auto sum_chunk = [&](const Frag<T> (&pf)[TPW][2], f32x4 (&lacc)[TPW]) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) mma(lacc[qt], ones, pf[qt][s2]);
  };
  // an LDS barrier that no instruction is scheduled across
  auto seg_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The pipeline of one phase over n chunks. stage_(y, commit): issue the
  // loads of D(y) (commit = false) or store them into their slots (true);
  // qk_(x): Q.K products of chunk x into st; seg1_(x): softmax arithmetic of
  // chunk x into pf; seg2_(x): the products of chunk x that use pf.
  auto run_phase = [&](int n, auto&& stage_, auto&& qk_, auto&& seg1_, auto&& seg2_) __attribute__((always_inline)) {
    stage_(0, false);
    stage_(0, true);
    stage_(1, false);
    stage_(1, true);
    seg_barrier();
    qk_(0);
    if (trail) seg_barrier();
#pragma unroll 1
    for (int x = 0; x < n; ++x) {
      const int y = trail ? x + 2 : x + 1;
      const bool stg_y = y >= 2 && y <= n;
      if (stg_y) stage_(y, false);
      seg1_(x);
      if (stg_y) stage_(y, true);
      seg_barrier();
      // the wave feeding the matrix unit goes first; its partner's vector
      // work fills the issue slots between the products
      __builtin_amdgcn_s_setprio(2);
      seg2_(x);
      if (x + 1 < n) qk_(x + 1);
      __builtin_amdgcn_s_setprio(0);
      seg_barrier();
    }
    if (!trail) seg_barrier();
  };
  const std::integral_constant<bool, true> kT{};
  const std::integral_constant<bool, false> kF{};
  bool nolo[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) nolo[qt] = false;
  f32x4 st[TPW][4], zero4[TPW];
  Frag<T> pf[TPW][2];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) zero4[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the compressed gate is applied once at the end: the accumulators carry
  // gate_win O_win / gc + P . Vc, then are scaled by gc (gc > 0 stands in for
  // a zero gate, whose branch then contributes 2^-30 of its output)
  float gc[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) gc[qt] = fmaxf(gcmp[qt], 0x1p-30f);

  // ---- sliding window over the workgroup's band of key blocks
  {
    const S* KT = static_cast<const S*>(a.kt) + bgoff * a.Nb * TILE;
    const S* VT = static_cast<const S*>(a.vt) + bgoff * a.Nb * TILE;
    const int b0 = max(0, T0 - a.w + 1) >> 6, b1 = Tl >> 6, nb = b1 - b0 + 1;
    float mw[TPW], alpha_w[TPW];
    f32x4 lw[TPW];
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      mw[qt] = kNegBig;
      lw[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // inner blocks [lo, hi]: inside the window of every token of the
    // workgroup (64 blk >= last token + 1 - w and 64 blk + 63 <= first token)
    int lo = b1 + 1, hi = b1;
    if (T0 + TPW * NW - 1 < Le) {
      const int x = T0 + TPW * NW - a.w;  // lowest first key of an inner block
      lo = x <= 0 ? b0 : max(b0, (x + 63) >> 6);
      hi = T0 >= 63 ? min(b1, (T0 - 63) >> 6) : -1;
      if (lo > hi) lo = hi + 1;
    }
    auto stage_w = [&](int y, bool commit) __attribute__((always_inline)) {
      const int64_t yk = b0 + min(y, nb - 1), yv = b0 + max(min(y - 1, nb - 1), 0);
      S* sl = stage + (y & 1) * BUF;
      S* slv = stage + ((y + 1) & 1) * BUF + TILE;
      if (y == 0) {
        if (!commit)
          stg.issue(KT + yk * TILE, VT + yk * TILE, nullptr, tid);
        else
          stg.commit(sl, sl + TILE, nullptr, tid);
      } else if (!commit) {
        stg.issue(KT + yk * TILE, y == 1 ? nullptr : VT + yv * TILE, nullptr, tid);
      } else {
        stg.commit(sl, y == 1 ? nullptr : slv, nullptr, tid);
      }
    };
    auto qk_w = [&](int x) __attribute__((always_inline)) { qk_chunk(stage + (x & 1) * BUF, nullptr, nolo, zero4, st); };
    // keys outside a token's window [t - w + 1, t] are masked on the edge
    // blocks; the running maxima rise lazily (kLazyMax), so the rescale is rare
    auto sm_w = [&](auto mask_c, int blk) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_c)::value;
      float lmx[TPW];
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
        const int t = tw + qt, klo = t - a.w + 1, khi = t < Le ? t : -1;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = st[qt][kt][i];
            if constexpr (MASK) {  // key 64 blk + 16 kt + i + g4 inside [klo, khi]; bounds uniform
              const int kb = 64 * blk + 16 * kt + i;
              x = (g4 >= klo - kb && g4 <= khi - kb) ? x : -INFINITY;
            }
            st[qt][kt][i] = x;
            mx = fmaxf(mx, x);
          }
        lmx[qt] = fmaxf(mx * sl2, kNegBig);
      }
      // each token decides alone (its wave partner differs between tilings
      // of the query rows, and the rows must not depend on the tiling); the
      // accumulators are rescaled in segment 2, ahead of the products
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
        alpha_w[qt] = 1.f;
        if (wave_any(lmx[qt] > mw[qt] + kLazyMax)) {
          const float mn = fmaxf(mw[qt], col_max4(lmx[qt]));
          alpha_w[qt] = fast_exp2(mw[qt] - mn);
          lw[qt] *= alpha_w[qt];
          mw[qt] = mn;
        }
      }
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[qt][kt][i] = fast_exp2(fmaf(st[qt][kt][i], sl2, -mw[qt]));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) pf[qt][s2] = pack_p<T>(st[qt][2 * s2], st[qt][2 * s2 + 1]);
      }
    };
    auto seg1_w = [&](int x) __attribute__((always_inline)) {
      const int blk = b0 + x;
      if (blk >= lo && blk <= hi)
        sm_w(kF, blk);
      else
        sm_w(kT, blk);
    };
    auto seg2_w = [&](int x) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt)
        if (wave_any(alpha_w[qt] != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] *= alpha_w[qt];
        }
      pv_chunk(stage + (x & 1) * BUF + TILE, pf, &lw);
    };
    run_phase(nb, stage_w, qk_w, seg1_w, seg2_w);
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const float lt = lw[qt][0];
      const float f = lt > 0.f ? gwin[qt] / (lt * gc[qt]) : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] *= f;
    }
  }

  // ---- compressed branch. The tiles of the block means of K hold them
  // scaled by softmax_scale * log2(e), so Q.K products are log2-domain logits.
  const int nch = (nvis_of(a, Tl) + 63) >> 6;
  const S* KC = static_cast<const S*>(a.kct) + bgoff * a.NcT * TILE;
  const S* KCL = kSplitKc<T> ? static_cast<const S*>(a.kclt) + bgoff * a.NcT * TILE : nullptr;
  const S* VC = static_cast<const S*>(a.vct) + bgoff * a.NcT * TILE;
  // chunks [0, nfull) are visible to both tokens in full (no masks)
  const int nfull = __builtin_amdgcn_readfirstlane(min(nch, nvis[0] >> 6));

  // pass 1: log-sum-exp (log2 domain) from the high part of the block means.
  // An error e_h in a head's log-sum-exp scales all of that head's
  // probabilities by exp(-e_h); the differences between block scores, which
  // the selection compares, move only in second order. The logits are kept
  // relative to a per-head offset m (the products start from -m), which
  // rises lazily; the sums run on the matrix unit.
  float lse2[TPW];
  if (nch > 0) {
    float m[TPW];
    f32x4 negm[TPW], l1[TPW];
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      m[qt] = 0.f;
      negm[qt] = zero4[qt];
      l1[qt] = zero4[qt];
    }
    auto stage_1 = [&](int y, bool commit) __attribute__((always_inline)) {
      if (!commit)
        stg.issue(KC + static_cast<int64_t>(min(y, nch - 1)) * TILE, nullptr, nullptr, tid);
      else
        stg.commit(stage + (y & 1) * BUF, nullptr, nullptr, tid);
    };
    auto qk_1 = [&](int x) __attribute__((always_inline)) {
      qk_chunk(stage + (x & 1) * BUF, nullptr, nolo, negm, st);
    };
    auto sm_1 = [&](auto full_c, int x) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_c)::value;
      float lmx[TPW];
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = (FULL || g4 < nvis[qt] - (64 * x + 16 * kt + i)) ? st[qt][kt][i] : -INFINITY;
            st[qt][kt][i] = v;
            mx = fmaxf(mx, v);
          }
        lmx[qt] = mx;
      }
      // raise the offsets: on the first chunk to its maxima (block 0 is
      // visible to every token that sees any block; one that sees none keeps
      // 0), later only when a logit passes the offset by kLazyMax (rare);
      // each token decides alone
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
        if (x == 0 || wave_any(lmx[qt] > kLazyMax)) {
          const float cm = col_max4(lmx[qt]);
          const float d = x == 0 ? (cm == -INFINITY ? 0.f : cm) : fmaxf(cm, 0.f);
          l1[qt] *= fast_exp2(-d);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) st[qt][kt] -= d;
          m[qt] += d;
          negm[qt] = f32x4{-m[qt], -m[qt], -m[qt], -m[qt]};
        }
      }
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[qt][kt][i] = fast_exp2(st[qt][kt][i]);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) pf[qt][s2] = pack_p<T>(st[qt][2 * s2], st[qt][2 * s2 + 1]);
      }
    };
    auto seg1_1 = [&](int x) __attribute__((always_inline)) {
      if (x < nfull)
        sm_1(kT, x);
      else
        sm_1(kF, x);
    };
    auto seg2_1 = [&](int) __attribute__((always_inline)) { sum_chunk(pf, l1); };
    run_phase(nch, stage_1, qk_1, seg1_1, seg2_1);
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) lse2[qt] = (nvis[qt] > 0 && colv) ? m[qt] + fast_log2(l1[qt][0]) : INFINITY;
  }

  // pass 2: probabilities (the products start from -lse), P . Vc into the
  // accumulators, block scores (computed even when the caller injects the
  // selection; they are then unused). The low parts of the means enter the
  // products only where a query sees fewer than kLoMinBlocks blocks or the
  // geometry is general.
  // the wave's two score rows: in LDS, or (GSC) the rows of its tokens in the
  // workspace (a wave past the last query row writes the spare rows)
  float* sc;
  if constexpr (GSC)
    sc = a.cmp_sc + ((static_cast<int64_t>(b) * a.G + g) * (a.Lq + 2) + min(tw - t0q, a.Lq)) * NcPad;
  else
    sc = scb + static_cast<size_t>(wave) * TPW * NcPad;
  if (nch > 0) {
    f32x4 negl[TPW];
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) negl[qt] = f32x4{-lse2[qt], -lse2[qt], -lse2[qt], -lse2[qt]};
    // The low parts are added by a token iff it sees fewer than kLoMinBlocks
    // blocks (or the geometry is general), never by the tiling of the query
    // rows; the workgroup stages them in LDS (slo) if any of its tokens adds
    // them. A token past the last query row follows token 0 of its wave; nvis
    // grows with the token, so lo[1] implies lo[0].
    bool lo[TPW];
    lo[0] = kSplitKc<T> && (!a.cmp_in_prep || nvis[0] < kLoMinBlocks);
    lo[1] = tw + 1 < Le ? kSplitKc<T> && (!a.cmp_in_prep || nvis[1] < kLoMinBlocks) : lo[0];
    const bool slo = kSplitKc<T> && LOLDS && (!a.cmp_in_prep || nvis_of(a, T0) < kLoMinBlocks);
    auto stage_2 = [&](int y, bool commit) __attribute__((always_inline)) {
      const int64_t yk = min(y, nch - 1), yv = max(min(y - 1, nch - 1), 0);
      S* sl = stage + (y & 1) * BUF;
      S* slv = stage + ((y + 1) & 1) * BUF + TILE;
      if (y == 0) {
        if (!commit)
          stg.issue(KC + yk * TILE, VC + yk * TILE, slo ? KCL + yk * TILE : nullptr, tid);
        else
          stg.commit(sl, sl + TILE, slo ? sl + 2 * TILE : nullptr, tid);
      } else if (!commit) {
        stg.issue(KC + yk * TILE, y == 1 ? nullptr : VC + yv * TILE, slo ? KCL + yk * TILE : nullptr, tid);
      } else {
        stg.commit(sl, y == 1 ? nullptr : slv, slo ? sl + 2 * TILE : nullptr, tid);
      }
    };
    auto qk_2 = [&](int x) __attribute__((always_inline)) {
      const S* kl = slo ? stage + (x & 1) * BUF + 2 * TILE : KCL + static_cast<int64_t>(x) * TILE;
      qk_chunk(stage + (x & 1) * BUF, kl, lo, negl, st);
    };
    auto sm_2 = [&](auto full_c, int x) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int qt = 0; qt < TPW; ++qt) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(st[qt][kt][i]);
            st[qt][kt][i] = (FULL || g4 < nvis[qt] - (64 * x + 16 * kt + i)) ? p : 0.f;
          }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const f32x4 pr[2] = {st[qt][2 * s2], st[qt][2 * s2 + 1]};
          // head sum of key 16·c₃ + 4·grp + 2·c₀ + c₁ of the half (c = col)
          sc[qt * NcPad + 64 * x + 32 * s2 + 16 * ((col >> 3) & 1) + 4 * grp + 2 * (col & 1) + ((col >> 1) & 1)] =
              row_scatter_sum8(pr, col);
          pf[qt][s2] = pack_p<T>(pr[0], pr[1]);
        }
      }
    };
    auto seg1_2 = [&](int x) __attribute__((always_inline)) {
      if (x < nfull)
        sm_2(kT, x);
      else
        sm_2(kF, x);
    };
    auto seg2_2 = [&](int x) __attribute__((always_inline)) { pv_chunk(stage + (x & 1) * BUF + TILE, pf, nullptr); };
    run_phase(nch, stage_2, qk_2, seg1_2, seg2_2);
  }
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] *= gc[qt];


  // ---- gate_win * O_win + gate_cmp * O_cmp -> out (fp32 output) or the fp32
  // partial rows (bf16 output); k_sel adds the selected branch, so a bf16
  // output is rounded once, from the fp32 sum of all three branches
  if constexpr (std::is_same<O, BF16>::value) {
    float* P = a.part + (static_cast<int64_t>(b) * a.Lq * a.Hq + h) * D + 4 * grp;
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = tw + qt;
      if (t < Le && colv) {
        float* o = P + static_cast<int64_t>(t - t0q) * a.Hq * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = oacc[qt][dt];
      }
    }
  } else {
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
    // score rows in the workspace: the wave's stores complete before its
    // lanes read each other's entries (the CU's L1 serves the reads)
    if constexpr (GSC) __threadfence_block();
    uint64_t* surv = survb + static_cast<size_t>(wave) * kSurvCap;
    int* selb = selbb + wave * 64;
#pragma unroll 1
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = tw + qt;
      if (t >= Le) break;
      int32_t* row = a.idx + ((static_cast<int64_t>(b) * a.Lq + (t - t0q)) * a.G + g) * a.n;
      const int own = t / a.ls;
      if (a.sel_map) {
        map_selection_scores(a, sc + qt * NcPad, own, nvis[qt], lane);
        if constexpr (GSC) __threadfence_block();
      }
      topk_wave(sc + qt * NcPad, own, a.n, row, surv, selb, lane);
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
template <class T, class O, int D, bool SAVE, bool PF>
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
  const int nwords = ((tl >> 5) + 4) >> 2;  // half blocks 0 .. tl / 32
  for (int w = lane; w < nwords; w += 64) bm[w] = 0u;
  // reads at clamped (token, head) indices, all issued before the first LDS
  // store, zeroed where not valid; the selected branch's gates are read now
  // rather than after the loop
  const S* Qc = static_cast<const S*>(a.q) + b * a.qs[0] + (colv ? h : g * a.Hg) * a.qs[2] + 8 * grp;
  Frag<T> qv[TPW][KS];
  float gsl[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt, tc = min(t, Le - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qv[qt][s] = frag_load_if<T>(Qc + static_cast<int64_t>(tc - t0q) * a.qs[1] + 32 * s, t < Le && colv);
  }
  {
    int rows[TPW];
    float gv[TPW][1];
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) rows[qt] = min(t0 + qt, Le - 1) - t0q;
    gates_of<T>(a, b, rows, colv ? h : g * a.Hg, {1}, gv);
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) gsl[qt] = t0 + qt < Le && colv ? gv[qt][0] : 0.f;
  }
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4* w = reinterpret_cast<const u32x4*>(&qv[qt][s]);
#pragma unroll
      for (int e = 0; e < FE; ++e) q_lds[wave][qt][s][e][lane] = w[e];
    }
  // the tokens' selection rows, both read before either is used
  int jv[TPW];
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int tc = min(t0 + qt, Le - 1);
    const int32_t* row = a.idx + ((static_cast<int64_t>(b) * a.Lq + (tc - t0q)) * a.G + g) * n;
    const int v = row[min(lane, n - 1)];
    jv[qt] = lane < n ? v : -1;
  }
  wave_lds_sync();
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    if (t >= Le) break;
    const int own = t / a.ls;
    const int j = jv[qt];
    if (j >= 0 && j <= own) {  // padding / unusable injected entries drop out
      // the selection block's half blocks that start at or before t
      const uint32_t bit = 1u << qt;
      const int hpb = a.ls >> 5, hb0 = j * hpb, hb1 = min(hb0 + hpb, (t >> 5) + 1);
      for (int hb = hb0; hb < hb1; ++hb) atomicOr(&bm[hb >> 2], bit << (8 * (hb & 3)));
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

  // The fp32 rows the epilogue adds to (the window + compressed part: partial
  // rows for a bf16 output, the output itself for fp32), copied to LDS by
  // direct global-to-LDS loads (lane l's 16 bytes land at slot l) issued just
  // before the ring's first loads, so the epilogue does not wait on memory.
  constexpr bool kPart = std::is_same<O, BF16>::value;
  float* pf = reinterpret_cast<float*>(sel_dyn + 4 * (static_cast<size_t>(a.sel_bm_words) + TPW * 128) * 4) +
              static_cast<size_t>(wave) * TPW * 16 * D;
  auto row_src = [&](int t, int hh) -> const float* {   // head g*Hg + hh of position t
    return kPart ? a.part + ((static_cast<int64_t>(b) * a.Lq + (t - t0q)) * a.Hq + g * a.Hg + hh) * D
                 : reinterpret_cast<const float*>(a.out) + b * a.os[0] + static_cast<int64_t>(t - t0q) * a.os[1] +
                       (g * a.Hg + hh) * a.os[2];
  };
  auto prefetch_rows = [&]() {
    if (!PF) return;
    const int nch = a.Hg * (D / 4);   // 16-byte chunks of one position's rows
#pragma unroll
    for (int qt = 0; qt < TPW; ++qt) {
      const int t = t0 + qt;
      if (t >= Le) break;
      for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        if (c < nch)
          lds_copy16(row_src(t, c / (D / 4)) + 4 * (c % (D / 4)), pf + qt * 16 * D + 4 * c0);
      }
    }
  };

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
  int code0[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) code0[k] = steps[max(0, min(k, nsteps - 1))];
  prefetch_rows();
  __builtin_amdgcn_sched_barrier(0);
  if (nsteps > 0) {
    HalfBlock<T, D> ring[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      half_load<T, D>(ring[k], KT, VT, code0[k] & 0x7FFFFF, (code0[k] >> 23) & 1, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      // loads return in order: once no more than the ring's loads are
      // outstanding, the prefetched rows are in LDS (and the compiler, seeing
      // this wait on every path, adds none of its own for them in the loop)
      constexpr int kRingLoads = NB * (2 * (D / 32) + D / 16) * FE;
      constexpr int kVm = kRingLoads < 63 ? kRingLoads : 63;
      __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
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

  SO* OUT = static_cast<SO*>(a.out) + b * a.os[0] + h * a.os[2] + 4 * grp;
#pragma unroll
  for (int qt = 0; qt < TPW; ++qt) {
    const int t = t0 + qt;
    const float lt = col_sum4(l[qt]);
    if (t < Le && colv) {
      const float f = lt > 0.f ? gsl[qt] / lt : 0.f;
      SO* o = OUT + static_cast<int64_t>(t - t0q) * a.os[1];
      // the window + compressed part (prefetched, or fp32 partial rows for a
      // bf16 output, out itself for fp32), all read before the first store:
      // the compiler cannot tell that the stores do not alias them, and would
      // otherwise wait for each read after the previous store
      f32x4 prev[DT];
      if (PF) {
        const float* pl = pf + qt * 16 * D + col * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) prev[dt] = *reinterpret_cast<const f32x4*>(pl + 16 * dt);
      } else if (kPart) {
        const float* pg = row_src(t, col) + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) prev[dt] = *reinterpret_cast<const f32x4*>(pg + 16 * dt);
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) prev[dt] = load4<O>(o + 16 * dt);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store4<O>(o + 16 * dt, prev[dt] + acc[qt][dt] * f);
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

size_t sel_lds_bytes(int Nb, int D, bool bf16, bool prefetch) {
  const size_t need = 4 * (static_cast<size_t>(sel_bm_words(Nb)) + kSelTPW * 128) * sizeof(uint32_t) +
                      (prefetch ? sel_pf_bytes(D) : 0);
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

template <class T, class O, int D>
// The 8-wave form (its two-segment schedule); score rows in LDS, or in the
// workspace when 8 waves' rows do not fit.
static const void* cmpwin_kernel(const PrefillArgs& a) {
  if (a.cmp_sc != nullptr)
    return a.cmp_lo_lds ? reinterpret_cast<const void*>(&k_cmpwin<T, O, D, 8, true, true>)
                        : reinterpret_cast<const void*>(&k_cmpwin<T, O, D, 8, false, true>);
  return a.cmp_lo_lds ? reinterpret_cast<const void*>(&k_cmpwin<T, O, D, 8, true, false>)
                      : reinterpret_cast<const void*>(&k_cmpwin<T, O, D, 8, false, false>);
}

static hipError_t launch_one(const void* fn, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                             const PrefillArgs& a) {
  void* args[] = {const_cast<PrefillArgs*>(&a)};
  return hipLaunchKernel(fn, grid, block, args, lds, st);
}

template <class T, class O, int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st, hipEvent_t* ev) {
  constexpr bool kBf16 = sizeof(typename T::storage) == 2;
  // every kernel attribute is set before the first launch
  const void* cmp_fn = cmpwin_kernel<T, O, D>(a);
  const size_t cmp_lds = cmpwin_lds_bytes(a.cmp_waves, a.cmp_sc != nullptr ? 0 : a.NcT, D, kBf16, a.cmp_lo_lds != 0);
  const void* sel_fn =
      a.save_o != nullptr
          ? (a.sel_pf ? reinterpret_cast<const void*>(&k_sel<T, O, D, true, true>)
                      : reinterpret_cast<const void*>(&k_sel<T, O, D, true, false>))
          : (a.sel_pf ? reinterpret_cast<const void*>(&k_sel<T, O, D, false, true>)
                      : reinterpret_cast<const void*>(&k_sel<T, O, D, false, false>));
  // Static + dynamic LDS above half a CU's caps residency at one workgroup
  // (4 waves) per CU, which was measured faster (~13 % at 64k) than two: the
  // gathers then contend less for L2.
  const size_t sel_lds = sel_lds_bytes(a.Nb, D, kBf16, a.sel_pf != 0);
  hipError_t e;
  if ((e = hipFuncSetAttribute(cmp_fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(cmp_lds))) !=
          hipSuccess ||
      (e = hipFuncSetAttribute(sel_fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sel_lds))) !=
          hipSuccess)
    return e;
  // workgroups per XCD (see the item mapping in k_sel)
  int per = a.sel_interleave ? a.B * ((a.sel_tiles + 8 / a.G - 1) / (8 / a.G)) : (a.B * a.G * a.sel_tiles + 7) / 8;
  if (!a.sel_interleave && a.sel_bounds[0] >= 0) {
    per = 0;
    for (int k = 0; k < 8 / a.G; ++k) per = max(per, a.sel_bounds[k + 1] - a.sel_bounds[k]);
  }
  const int nblk_prep = a.cmp_in_prep ? max(a.Nb, a.NcT * 64) : a.Nb;
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  if (a.gate_w != nullptr) {
    const int64_t rows = static_cast<int64_t>(a.B) * a.Lq * a.Hq;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((rows + 255) / 256, 65536));
    if ((e = launch_one(reinterpret_cast<const void*>(&k_gate<T, D>), dim3(grid), dim3(256), 0, st, a)) !=
        hipSuccess)
      return e;
  }
  if ((e = launch_one(reinterpret_cast<const void*>(&k_prep<T, D>), dim3(nblk_prep, a.G, a.B), dim3(256), 0, st,
                      a)) != hipSuccess)
    return e;
  if (!a.cmp_in_prep && a.NcT > 0 &&
      (e = launch_one(reinterpret_cast<const void*>(&k_ctile<T, D>), dim3(2 * a.NcT, a.G, a.B), dim3(256), 0, st,
                      a)) != hipSuccess)
    return e;
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  if ((e = launch_one(cmp_fn, dim3(a.B * a.G * a.cmp_tiles), dim3(64 * a.cmp_waves), cmp_lds, st, a)) != hipSuccess)
    return e;
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
  if ((e = launch_one(sel_fn, dim3(per * 8), dim3(256), sel_lds, st, a)) != hipSuccess) return e;
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
