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
//  k_dsa_topk   one workgroup per query row: an exact radix select of the
//               top-k (12 + 12 + 8 bits of an order-preserving key; the row
//               cached in LDS up to a capacity), ties to the lower token,
//               then an ordered ballot compaction that writes the chosen
//               tokens ascending, padded with -1.
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
// fragment of d-tile dt for lane l is 8 contiguous elements at (dt*64 + l)*8
// holding V[kappa(l/16, j)][16 dt + l%16] (kappa as for the 64-key V^T tiles:
// the keys whose probabilities lane l holds after the S^T product).
__device__ __forceinline__ int vhalf_off(int r, int d) {
  const int half = r >> 4, a = (r & 15) >> 2, i = r & 3;
  const int lane = (d & 15) + 16 * a;
  return ((d >> 4) * 64 + lane) * 8 + 4 * half + i;
}
__device__ __forceinline__ int vhalf_frag(int dt, int lane) { return (dt * 64 + lane) * 8; }

// Unsigned key that orders like the float (larger float -> larger key).
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ k_dsa_index

constexpr int kIdxWaves = 8, kIdxTPW = 2;

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
#pragma unroll
  for (int qt = 0; qt < kIdxTPW; ++qt) {
    const int t = tw + qt;
    const bool ok = t < a.L && col < a.Hi;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = ok ? frag_load<T>(QI + static_cast<int64_t>(t) * a.qis[1] + col * a.qis[2] + 32 * s + 8 * grp)
                     : frag_zero<T>();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      wv[qt][i] = (t < a.L && h < a.Hi) ? to_f32<T>(W[static_cast<int64_t>(t) * a.wis[1] + h]) : 0.f;
    }
  }

  // 16-byte chunk e of chunk c: key row r, dims d .. d + EPC - 1 -> its place in the fragment-major tile
  u32x4 reg[PER];
  auto issue = [&](int c) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NT * i, r = (e * EPC) / DI, d = (e * EPC) % DI, key = 64 * c + r;
      reg[i] = key < a.L ? *reinterpret_cast<const u32x4*>(KI + static_cast<int64_t>(key) * a.kis[1] + d)
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NT * i, r = (e * EPC) / DI, d = (e * EPC) % DI;
      *reinterpret_cast<u32x4*>(&stage[buf][ktile_off(r, d, DI)]) = reg[i];
    }
  };
  const int nch = (Tl >> 6) + 1;
  issue(0);
  commit(0);
  __syncthreads();
  float* SC = a.scores;
  int64_t rows[kIdxTPW];
#pragma unroll
  for (int qt = 0; qt < kIdxTPW; ++qt) rows[qt] = score_row(a, b, min(tw + qt, a.L - 1));
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) issue(c + 1);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      Frag<T> kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = frag_load<T>(&stage[buf][ktile_frag(kt, s, lane, DI)]);
      const int key = 64 * c + 16 * kt + col;
#pragma unroll
      for (int qt = 0; qt < kIdxTPW; ++qt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(acc, qf[qt][s], kf[s]);
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wv[qt][i], fmaxf(acc[i], 0.f), v);
        // heads 4 grp .. 4 grp + 3 of the four lanes of this column; + 0 turns -0 into +0
        v = col_sum4(v) + 0.f;
        const int t = tw + qt;
        if (grp == 0 && t < a.L && key <= t) SC[rows[qt] + key] = v;
      }
    }
    if (more) commit(buf ^ 1);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ k_dsa_topk

constexpr int kTopkThreads = 512;

// The bin holding the `need`-th largest element (1-based) of a histogram of
// nb bins, and that element's rank inside the bin. Wave 0 computes it; the
// caller synchronises afterwards.
__device__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* lane_tot, uint32_t* result, int tid) {
  if (tid < 64) {
    const int per = nb / 64, lo = tid * per;
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i) sum += hist[lo + i];
    lane_tot[tid] = sum;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    uint32_t above = 0;  // elements in the bins of higher lanes
    for (int j = tid + 1; j < 64; ++j) above += lane_tot[j];
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = hist[lo + i];
      if (above < need && need <= above + c) {
        result[0] = static_cast<uint32_t>(lo + i);
        result[1] = need - above;
      }
      above += c;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void k_dsa_topk(DsaArgs a) {
  extern __shared__ __align__(16) uint32_t tk_lds[];
  uint32_t* hist = tk_lds;           // 4096 bins
  uint32_t* cache = tk_lds + 4096;   // orderable keys of the row's first topk_cache candidates
  __shared__ uint32_t lane_tot[64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t wcnt[2][2][kTopkThreads / 64];  // [round parity][greater, equal][wave]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / a.L), t = static_cast<int>(row % a.L);
  const int n = t + 1, k = a.topk;
  int32_t* out = a.idx + row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* S = a.scores + score_row(a, b, t);
  const int nc = min(n, a.topk_cache);
  auto key_at = [&](int i) -> uint32_t { return i < nc ? cache[i] : orderable(S[i]); };

  // digit 1: bits 31..20
  for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t u = orderable(S[i]);
    if (i < nc) cache[i] = u;
    atomicAdd(&hist[u >> 20], 1u);
  }
  __syncthreads();
  find_bin(hist, 4096, static_cast<uint32_t>(k), lane_tot, res, tid);
  __syncthreads();
  const uint32_t d1 = res[0], need1 = res[1];
  // digit 2: bits 19..8 of the keys in bin d1
  for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t u = key_at(i);
    if ((u >> 20) == d1) atomicAdd(&hist[(u >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  find_bin(hist, 4096, need1, lane_tot, res, tid);
  __syncthreads();
  const uint32_t pre = (d1 << 12) | res[0], need2 = res[1];
  // digit 3: bits 7..0 of the keys sharing the first 24 bits
  for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t u = key_at(i);
    if ((u >> 8) == pre) atomicAdd(&hist[u & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin(hist, 256, need2, lane_tot, res, tid);
  __syncthreads();
  // the k-th largest key, and how many of the keys equal to it are taken
  // (those of the lowest tokens: ties go to the lower token)
  const uint32_t ustar = (pre << 8) | res[0], quota0 = res[1];

  // ordered compaction in rounds of kTopkThreads candidates
  uint32_t written = 0, ties_seen = 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int r0 = 0, par = 0; r0 < n; r0 += kTopkThreads, par ^= 1) {
    const int i = r0 + tid;
    const uint32_t u = i < n ? key_at(i) : 0u;
    const bool gt = i < n && u > ustar, eq = i < n && u == ustar;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      wcnt[par][0][wave] = static_cast<uint32_t>(__popcll(bg));
      wcnt[par][1][wave] = static_cast<uint32_t>(__popcll(be));
    }
    __syncthreads();
    uint32_t gt_before = static_cast<uint32_t>(__popcll(bg & below)), eq_before = static_cast<uint32_t>(__popcll(be & below));
    uint32_t gt_tot = 0, eq_tot = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      if (w < wave) {
        gt_before += wcnt[par][0][w];
        eq_before += wcnt[par][1][w];
      }
      gt_tot += wcnt[par][0][w];
      eq_tot += wcnt[par][1][w];
    }
    const uint32_t quota = quota0 > ties_seen ? quota0 - ties_seen : 0u;  // ties still to take
    const bool take = gt || (eq && eq_before < quota);
    if (take) out[written + gt_before + min(eq_before, quota)] = i;
    written += gt_tot + min(eq_tot, quota);
    ties_seen += eq_tot;
  }
}

// ------------------------------------------------------------------ k_dsa_attn

template <class T, class O, int D, int WPG>
__global__ __launch_bounds__(256) void k_dsa_attn(DsaArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int KS = D / 32, DT = D / 16, HALF = 32 * D;   // elements of a 32-key K piece or V^T piece
  constexpr int EPC = 16 / static_cast<int>(sizeof(S));
  constexpr int CH = HALF / EPC;                             // 16-byte chunks of a piece
  extern __shared__ __align__(16) unsigned char at_lds[];
  __shared__ int cnt_sh;
  __shared__ uint32_t wtot[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NTH = 64 * a.waves;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / a.L), t = static_cast<int>(row % a.L);
  constexpr int wpg = WPG;                      // waves sharing one KV head (Hg / 16, or 1)
  const int ngw = a.waves / wpg;                 // KV heads in the workgroup (= G)
  const int gw = wave / wpg;
  const int h0 = a.Hg >= 16 ? 16 * wave : gw * a.Hg;
  const int col = lane & 15, grp = lane >> 4;
  const bool colv = col < a.heads_per_wave;
  S* gbuf = reinterpret_cast<S*>(at_lds) + static_cast<size_t>(gw) * 4 * HALF;   // [2 buffers][K, V^T]
  int* list = reinterpret_cast<int*>(at_lds + static_cast<size_t>(ngw) * 4 * HALF * sizeof(S));
  int P = 1;
  while (P < a.topk) P <<= 1;
  int* tmp = list + P;

  // ---- this token's keys: ascending, distinct, each at or before t
  const int32_t* irow = a.idx + row * a.topk;
  if (tid == 0) cnt_sh = 0;
  __syncthreads();
  if (!a.inject) {
    // a computed row is ascending with -1 padding
    int c = 0;
    for (int i = tid; i < a.topk; i += NTH) {
      const int j = irow[i];
      list[i] = j;
      c += j >= 0 ? 1 : 0;
    }
    if (c) atomicAdd(&cnt_sh, c);
    __syncthreads();
  } else {
    // an injected row is a set of tokens: drop entries outside [0, t], sort, drop repeats
    for (int i = tid; i < P; i += NTH) {
      const int j = i < a.topk ? irow[i] : -1;
      tmp[i] = (j >= 0 && j <= t) ? j : INT_MAX;
    }
    __syncthreads();
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
        __syncthreads();
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
      __syncthreads();
      int before = __popcll(bal & below), tot = 0;
      for (int w = 0; w < a.waves; ++w) {
        if (w < wave) before += static_cast<int>(wtot[w]);
        tot += static_cast<int>(wtot[w]);
      }
      if (keep) list[written + before] = x;
      written += tot;
      __syncthreads();
    }
    if (tid == 0) cnt_sh = written;
    __syncthreads();
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
  u32x4 rk[MAXPER], rv[MAXPER];
  auto issue = [&](int step) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int e = gt + gthreads * i;
      rk[i] = rv[i] = u32x4{0u, 0u, 0u, 0u};
      if (e < CH) {
        const int r = (e * EPC) / D, d = (e * EPC) % D, pos = 32 * step + r;
        if (pos < cnt) {
          const int64_t tok = list[pos];
          rk[i] = *reinterpret_cast<const u32x4*>(K + tok * a.ks[1] + d);
          rv[i] = *reinterpret_cast<const u32x4*>(V + tok * a.vs[1] + d);
        }
      }
    }
  };
  auto commit = [&](int buf) {
    S* kp = gbuf + buf * 2 * HALF;
    S* vp = kp + HALF;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int e = gt + gthreads * i;
      if (e < CH) {
        const int r = (e * EPC) / D, d = (e * EPC) % D;
        *reinterpret_cast<u32x4*>(kp + ktile_off(r, d, D)) = rk[i];
        const S* src = reinterpret_cast<const S*>(&rv[i]);
#pragma unroll
        for (int j = 0; j < EPC; ++j) vp[vhalf_off(r, d + j)] = src[j];
      }
    }
  };

  const float sl2 = a.scale_log2;
  float m = kNegBig, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsteps = (cnt + 31) >> 5;
  if (nsteps > 0) {
    issue(0);
    commit(0);
    __syncthreads();
  }
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) issue(step + 1);
    const S* kp = gbuf + buf * 2 * HALF;
    const S* vp = kp + HALF;
    f32x4 st[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      st[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) mma(st[h2], frag_load<T>(kp + ktile_frag(h2, s, lane, D)), qf[s]);
    }
    Frag<T> vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vp + vhalf_frag(dt, lane));
    // positions past the list hold zero rows: masked out of the softmax
    if (32 * step + 31 < cnt)
      online_step<T, DT, false>(st, 32 * step, 0, 0, grp, sl2, m, l, acc, vf);
    else
      online_step<T, DT, true>(st, 32 * step, 0, cnt - 1, grp, sl2, m, l, acc, vf);
    if (more) commit(buf ^ 1);
    __syncthreads();
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
  const void* topk = reinterpret_cast<const void*>(&k_dsa_topk);
  const size_t attn_lds = dsa_attn_lds_bytes(a.waves / wpg, D, kBf16, a.topk);
  const size_t topk_lds = dsa_topk_lds_bytes(a.topk_cache);
  hipError_t e;
  if ((e = hipFuncSetAttribute(attn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(attn_lds))) !=
          hipSuccess ||
      (e = hipFuncSetAttribute(topk, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(topk_lds))) !=
          hipSuccess)
    return e;
  const unsigned rows = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.L);
  if ((e = record(ev, 0, st)) != hipSuccess) return e;
  if (!a.inject &&
      (e = launch_one(reinterpret_cast<const void*>(&k_dsa_index<T, DI>), dim3(a.B * a.idx_tiles), dim3(512), 0,
                      st, a)) != hipSuccess)
    return e;
  if ((e = record(ev, 1, st)) != hipSuccess) return e;
  if (!a.inject && (e = launch_one(topk, dim3(rows), dim3(kTopkThreads), topk_lds, st, a)) != hipSuccess) return e;
  if ((e = record(ev, 2, st)) != hipSuccess) return e;
  if ((e = launch_one(attn, dim3(rows), dim3(64 * a.waves), attn_lds, st, a)) != hipSuccess) return e;
  if ((e = record(ev, 3, st)) != hipSuccess) return e;
  return hipGetLastError();
}

template <class T, class O>
hipError_t launch_dsa_o(const DsaArgs& a, hipStream_t st, hipEvent_t* ev) {
  if (a.D == 64) return a.Di == 64 ? launch_dsa_t<T, O, 64, 64>(a, st, ev) : launch_dsa_t<T, O, 64, 128>(a, st, ev);
  return a.Di == 64 ? launch_dsa_t<T, O, 128, 64>(a, st, ev) : launch_dsa_t<T, O, 128, 128>(a, st, ev);
}

}  // namespace

size_t dsa_topk_lds_bytes(int cache) { return (4096 + static_cast<size_t>(cache)) * sizeof(uint32_t); }

size_t dsa_attn_lds_bytes(int groups_per_wg, int D, bool bf16, int k) {
  int P = 1;
  while (P < k) P <<= 1;
  return static_cast<size_t>(groups_per_wg) * 4 * 32 * D * (bf16 ? 2 : 4) + 2 * static_cast<size_t>(P) * sizeof(int);
}

hipError_t launch_dsa(const DsaArgs& a, bool in_bf16, bool out_bf16, hipStream_t st, hipEvent_t* ev) {
  if (in_bf16) return out_bf16 ? launch_dsa_o<BF16, BF16>(a, st, ev) : launch_dsa_o<BF16, F32>(a, st, ev);
  return launch_dsa_o<F32, F32>(a, st, ev);
}

}  // namespace nsa
