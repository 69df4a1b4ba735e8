// Backward pass of the NSA prefill: dq, dk, dv and the gate gradients for a
// fixed block selection (the top-k choice carries no gradient).
//
// NSA is trained end to end and its backward pass is claimed to speed up with
// the same sparsity as the forward (NSA how-to, qwbw.cn/news/106443, section
// 1). Each branch is softmax attention over its key set, so its gradients are
// the textbook ones: with P the probabilities, o the branch output and
// g its gate, dgate = dout.o, dS = g P (dout.V^T - dout.o),
// dq = scale dS K, dK = scale dS^T q, dV = g P^T dout. The compressed
// branch's keys are block means, so their gradients reach each token of the
// block divided by 64.
//
// Kernels, in launch order:
//   k_bzero   clears the accumulated gradients and the selection counters;
//   k_compress (shared with nsa_compress_kv) forms the block means;
//   k_btile   re-lays K, V and the means into 64-key tiles, twice each: the
//             fragment-major layout (operand of S = q.K^T and dP = dout.V^T)
//             and the V^T layout (operand of O^T = V^T P^T and dq^T = K^T dS^T);
//   k_btrans  writes q and dout head-minor ([token][group][d][16 heads]), the
//             operand layout of the key-side products dK = dS^T q and
//             dV = P^T dout, and a compact copy of dout in the input type;
//   k_bsel_count / k_bsel_scan / k_bsel_fill
//             invert the selection: for each (sequence, group, block), the
//             tokens that chose it;
//   k_bq      query side, one wave per (token, group): for each branch, the
//             forward over its key set (log-sum-exp and dout.o, which is also
//             the gate gradient), then dq; with the selected branch's output
//             and log-sum-exp kept by the forward (nsa_fwd_prefill_save),
//             that branch skips its forward and gathers its blocks once;
//   k_bkv     key side, one workgroup per (branch, group, 64-key block,
//             piece of its token set), each wave a 16-key tile: dK and dV
//             accumulated over the tokens that see the block (staged through
//             LDS a few at a time for the four waves), then added to the fp32
//             outputs with atomics;
//   k_bfin    adds the block-mean gradients / 64 to the tokens of each block.
#include <algorithm>

#include "nsa_device.h"
#include "nsa_backward.h"

namespace nsa {

namespace {

__global__ __launch_bounds__(256) void k_bzero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(256) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = 0u;
}

// One 64-row chunk of src (rows [64c, 64c + 64) of group g of sequence b,
// element (b, r, g, d) at b*s0 + r*s1 + g*s2 + d) -> the fragment-major tile
// and the V^T tile of that chunk. Rows at or past `rows` are zero.
template <class T, int D>
__global__ __launch_bounds__(256) void k_btile(const typename T::storage* src, int64_t s0, int64_t s1,
                                               int64_t s2, int rows, int nchunk,
                                               typename T::storage* ta, typename T::storage* tv) {
  using S = typename T::storage;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const size_t base = ((static_cast<size_t>(b) * gridDim.y + g) * nchunk + c) * 64 * D;
  for (int e = threadIdx.x; e < 64 * D; e += 256) {
    const int r = e / D, d = e % D, row = c * 64 + r;
    const S x = row < rows ? src[b * s0 + row * s1 + g * s2 + d] : S{};
    ta[base + ktile_off(r, d, D)] = x;
    tv[base + vtile_off(r, d)] = x;
  }
}

// Per token: qT / dT [b][t][g][d][16] (head within the group fastest, zero
// past Hg) and dN [b][t][h][d], dout converted to the input type. One group
// at a time goes through LDS: 16-byte coalesced reads of its heads' rows,
// then the head-minor rows written in order.
template <class T, class O, int D>
__global__ __launch_bounds__(256) void k_btrans(BwdArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  __shared__ S qs[16][D], ds[16][D];
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const S* q = static_cast<const S*>(a.q) + b * a.qs[0] + t * a.qs[1];
  const SO* dout = static_cast<const SO*>(a.dout) + b * a.os[0] + t * a.os[1];
  const size_t row = static_cast<size_t>(b) * a.L + t;
  for (int g = 0; g < a.G; ++g) {
    __syncthreads();  // the previous group's rows have been read
    for (int e = tid * 8; e < 16 * D; e += 256 * 8) {
      const int hh = e / D, d = e % D;
      Frag<T> xq = frag_zero<T>(), xd = frag_zero<T>();
      if (hh < a.Hg) {
        const int h = g * a.Hg + hh;
        xq = frag_load<T>(q + h * a.qs[2] + d);
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = to_f32<O>(dout[h * a.os[2] + d + j]);
        S* dn = static_cast<S*>(a.dN) + (row * a.Hq + h) * D + d;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const S x = from_f32<T>(f[j]);
          ds[hh][d + j] = x;
          dn[j] = x;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) ds[hh][d + j] = S{};
      }
      frag_store<T>(&qs[hh][d], xq);
    }
    __syncthreads();
    S* qT = static_cast<S*>(a.qT) + (row * a.G + g) * D * 16;
    S* dT = static_cast<S*>(a.dT) + (row * a.G + g) * D * 16;
    for (int e = tid; e < 16 * D; e += 256) {
      const int hh = e & 15, d = e >> 4;
      qT[e] = qs[hh][d];
      dT[e] = ds[hh][d];
    }
  }
}

// Entry i of a selection row counts when it names a block at or before the
// token's own one and no earlier entry of the row names the same block (the
// selection is a set of blocks).
__device__ __forceinline__ bool sel_entry(const int32_t* row, int i, int own) {
  const int j = row[i];
  if (j < 0 || j > own) return false;
  for (int i2 = 0; i2 < i; ++i2)
    if (row[i2] == j) return false;
  return true;
}

__global__ __launch_bounds__(256) void k_bsel_count(BwdArgs a) {
  const int64_t id = blockIdx.x * static_cast<int64_t>(256) + threadIdx.x;
  if (id >= static_cast<int64_t>(a.B) * a.L * a.G) return;
  const int g = static_cast<int>(id % a.G), t = static_cast<int>((id / a.G) % a.L);
  const int b = static_cast<int>(id / (static_cast<int64_t>(a.G) * a.L));
  const int32_t* row = a.idx + id * a.n;
  int32_t* cnt = a.cnt + (static_cast<size_t>(b) * a.G + g) * a.Nb;
  for (int i = 0; i < a.n; ++i)
    if (sel_entry(row, i, t >> 6)) atomicAdd(cnt + row[i], 1);
}

// One workgroup per (sequence, group): offs = exclusive prefix of the counts,
// pofs = exclusive prefix of the pieces (ceil(count / kBwdSelPiece)); the
// counts are reset to serve as fill cursors.
__global__ __launch_bounds__(256) void k_bsel_scan(BwdArgs a) {
  __shared__ int part[256], ppart[256];
  const int bg = blockIdx.x, Nb = a.Nb;
  int32_t* cnt = a.cnt + static_cast<size_t>(bg) * Nb;
  int32_t* offs = a.offs + static_cast<size_t>(bg) * (Nb + 1);
  int32_t* pofs = a.pofs + static_cast<size_t>(bg) * (Nb + 1);
  const int per = (Nb + 255) / 256, j0 = threadIdx.x * per, j1 = min(Nb, j0 + per);
  int s = 0, ps = 0;
  for (int j = j0; j < j1; ++j) {
    s += cnt[j];
    ps += (cnt[j] + kBwdSelPiece - 1) / kBwdSelPiece;
  }
  part[threadIdx.x] = s;
  ppart[threadIdx.x] = ps;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0, prun = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = part[i], px = ppart[i];
      part[i] = run;
      ppart[i] = prun;
      run += x;
      prun += px;
    }
    offs[Nb] = run;
    pofs[Nb] = prun;
  }
  __syncthreads();
  s = part[threadIdx.x];
  ps = ppart[threadIdx.x];
  for (int j = j0; j < j1; ++j) {
    const int c = cnt[j];
    offs[j] = s;
    pofs[j] = ps;
    s += c;
    ps += (c + kBwdSelPiece - 1) / kBwdSelPiece;
    cnt[j] = 0;
  }
}

__global__ __launch_bounds__(256) void k_bsel_fill(BwdArgs a) {
  const int64_t id = blockIdx.x * static_cast<int64_t>(256) + threadIdx.x;
  if (id >= static_cast<int64_t>(a.B) * a.L * a.G) return;
  const int g = static_cast<int>(id % a.G), t = static_cast<int>((id / a.G) % a.L);
  const int b = static_cast<int>(id / (static_cast<int64_t>(a.G) * a.L));
  const int32_t* row = a.idx + id * a.n;
  const size_t bg = static_cast<size_t>(b) * a.G + g;
  int32_t* cur = a.cnt + bg * a.Nb;
  const int32_t* offs = a.offs + bg * (a.Nb + 1);
  int32_t* list = a.list + bg * static_cast<size_t>(a.L) * a.n;
  for (int i = 0; i < a.n; ++i)
    if (sel_entry(row, i, t >> 6)) {
      const int j = row[i];
      list[offs[j] + atomicAdd(cur + j, 1)] = t;
    }
}

// The key set of branch X for token t as a list of 64-key chunks: chunk i
// covers keys [base, base + 64) of tile `tile`, of which [klo, khi] count.
// X = 0 compressed (keys are block means), 1 selected, 2 window.
struct Chunk {
  int tile, base, klo, khi;
  bool ok;
};

template <int X>
__device__ __forceinline__ int n_chunks(const BwdArgs& a, int t) {
  if (X == 0) return (((t + 1) >> 6) + 63) >> 6;
  if (X == 1) return a.n;
  return (t >> 6) - (max(0, t - a.w + 1) >> 6) + 1;
}

template <int X>
__device__ __forceinline__ Chunk chunk_at(const BwdArgs& a, int t, const int32_t* row, int i) {
  Chunk c;
  if (X == 0) {
    c.tile = i;
    c.base = 64 * i;
    c.klo = 0;
    c.khi = ((t + 1) >> 6) - 1;
    c.ok = true;
  } else if (X == 1) {
    c.ok = sel_entry(row, i, t >> 6);
    const int j = c.ok ? row[i] : 0;
    c.tile = j;
    c.base = 64 * j;
    c.klo = 64 * j;
    c.khi = min(64 * j + 63, t);
  } else {
    const int lo = max(0, t - a.w + 1);
    c.tile = (lo >> 6) + i;
    c.base = 64 * c.tile;
    c.klo = lo;
    c.khi = t;
    c.ok = true;
  }
  return c;
}

// Query side of branch X for one token (one wave, 16 head columns): the
// forward over the key set (log-sum-exp, o, dout.o), then dq += scale dS K.
// SAVED (selected branch only): the branch's output and log-sum-exp come
// from the forward (BwdArgs::o_slc / lse_slc) instead of a forward pass here.
template <class T, class O, int D, int X, bool SAVED = false>
__device__ __forceinline__ void bq_branch(const BwdArgs& a, int b, int g, int t, int lane,
                                          const Frag<T> (&qf)[D / 32], const Frag<T> (&df)[D / 32],
                                          float gate, const typename O::storage* dout_row,
                                          f32x4 (&dq)[D / 16], float2* stat, float* dgate) {
  using S = typename T::storage;
  constexpr int KS = D / 32, DT = D / 16;
  const int col = lane & 15, grp = lane >> 4;
  const float sl2 = a.scale_log2;
  const size_t bg = static_cast<size_t>(b) * a.G + g;
  const S* KA = static_cast<const S*>(X == 0 ? a.kca : a.ka) + bg * (X == 0 ? a.NcT : a.Nb) * 64 * D;
  const S* VV = static_cast<const S*>(X == 0 ? a.vcv : a.vv) + bg * (X == 0 ? a.NcT : a.Nb) * 64 * D;
  const S* VA = static_cast<const S*>(X == 0 ? a.vca : a.va) + bg * (X == 0 ? a.NcT : a.Nb) * 64 * D;
  const S* KV = static_cast<const S*>(X == 0 ? a.kcv : a.kv) + bg * (X == 0 ? a.NcT : a.Nb) * 64 * D;
  const int32_t* row = a.idx + ((static_cast<size_t>(b) * a.L + t) * a.G + g) * a.n;
  const int nch = n_chunks<X>(a, t);

  float lse2 = 0.f, dsum = 0.f;
  bool any = false;
  if (SAVED) {
    for (int i = 0; i < nch && !any; ++i) any = chunk_at<X>(a, t, row, i).ok;
    if (any) {
      const size_t r = (static_cast<size_t>(b) * a.L + t) * a.Hq + g * a.Hg + (col < a.Hg ? col : 0);
      lse2 = a.lse_slc[r] * kLog2e;
      const typename O::storage* op = static_cast<const typename O::storage*>(a.o_slc) + r * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dsum += to_f32<O>(dout_row[16 * dt + 4 * grp + i]) * to_f32<O>(op[16 * dt + 4 * grp + i]);
      dsum = col_sum4(dsum);
    }
  } else {
  // forward over the key set
  float m = kNegBig, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nch; ++i) {
    const Chunk c = chunk_at<X>(a, t, row, i);
    if (!c.ok || c.khi < c.klo) continue;
    any = true;
    const S* kt = KA + static_cast<size_t>(c.tile) * 64 * D;
    const S* vt = VV + static_cast<size_t>(c.tile) * 64 * D;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int s = 0; s < KS; ++s) mma(st[h2], frag_load<T>(kt + ktile_frag(2 * s2 + h2, s, lane, D)), qf[s]);
      Frag<T> vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = frag_load<T>(vt + vtile_frag(dt, s2, lane));
      online_step<T, DT, true>(st, c.base + 32 * s2, c.klo, c.khi, grp, sl2, m, l, acc, vf);
    }
  }
  if (any) {
    const float lt = col_sum4(l);
    lse2 = m + fast_log2(lt);
    const float inv = 1.0f / lt;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dsum += to_f32<O>(dout_row[16 * dt + 4 * grp + i]) * acc[dt][i] * inv;
    dsum = col_sum4(dsum);
  }
  }
  if (grp == 0 && stat != nullptr) {
    stat[X] = make_float2(lse2, dsum);
    dgate[X] = dsum;
  }
  if (!any) return;

  // dq^T += K^T dS^T over the same key set
  for (int i = 0; i < nch; ++i) {
    const Chunk c = chunk_at<X>(a, t, row, i);
    if (!c.ok || c.khi < c.klo) continue;
    const S* kt = KA + static_cast<size_t>(c.tile) * 64 * D;
    const S* va = VA + static_cast<size_t>(c.tile) * 64 * D;
    const S* kv = KV + static_cast<size_t>(c.tile) * 64 * D;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          mma(st[h2], frag_load<T>(kt + ktile_frag(2 * s2 + h2, s, lane, D)), qf[s]);
          mma(dp[h2], frag_load<T>(va + ktile_frag(2 * s2 + h2, s, lane, D)), df[s]);
        }
      f32x4 ds[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int key = c.base + 32 * s2 + 16 * h2 + 4 * grp + i2;
          const float p = (key >= c.klo && key <= c.khi) ? fast_exp2(fmaf(st[h2][i2], sl2, -lse2)) : 0.f;
          ds[h2][i2] = gate * p * (dp[h2][i2] - dsum);
        }
      const Frag<T> dsf = pack_p<T>(ds[0], ds[1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mma(dq[dt], frag_load<T>(kv + vtile_frag(dt, s2, lane)), dsf);
    }
  }
}

// Three waves per SIMD (at most 168 registers, a few spilled) measured 9 %
// faster than the unconstrained two: each wave spends most of its time
// waiting for one gathered tile, so more waves hide more of that latency;
// four (128 registers) spilled too much and was 40 % slower.
template <class T, class O, int D, bool SAVED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_bq(BwdArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int KS = D / 32, DT = D / 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int tiles = (a.L + 3) >> 2;
  const int tile = static_cast<int>(blockIdx.x % tiles), bg = static_cast<int>(blockIdx.x / tiles);
  const int g = bg % a.G, b = bg / a.G;
  const int t = tile * 4 + wave;
  if (t >= a.L) return;
  const bool colv = col < a.Hg;
  const int h = g * a.Hg + (colv ? col : 0);
  const S* qp = static_cast<const S*>(a.q) + b * a.qs[0] + t * a.qs[1] + h * a.qs[2];
  const size_t row = static_cast<size_t>(b) * a.L + t;
  const S* dnp = static_cast<const S*>(a.dN) + (row * a.Hq + h) * D;
  Frag<T> qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = colv ? frag_load<T>(qp + 32 * s + 8 * grp) : frag_zero<T>();
    df[s] = colv ? frag_load<T>(dnp + 32 * s + 8 * grp) : frag_zero<T>();
  }
  const S* gp = static_cast<const S*>(a.gates) + b * a.gs[0] + t * a.gs[1] + h * a.gs[2];
  const float g0 = colv ? to_f32<T>(gp[0]) : 0.f, g1 = colv ? to_f32<T>(gp[1]) : 0.f,
              g2 = colv ? to_f32<T>(gp[2]) : 0.f;
  const SO* dout_row = static_cast<const SO*>(a.dout) + b * a.os[0] + t * a.os[1] + h * a.os[2];
  float2* stat = colv ? a.stat + (row * a.Hq + h) * 3 : nullptr;
  float* dgate = colv ? a.dgates + (row * a.Hq + h) * 3 : nullptr;
  f32x4 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bq_branch<T, O, D, 0>(a, b, g, t, lane, qf, df, g0, dout_row, dq, stat, dgate);
  bq_branch<T, O, D, 1, SAVED>(a, b, g, t, lane, qf, df, g1, dout_row, dq, stat, dgate);
  bq_branch<T, O, D, 2>(a, b, g, t, lane, qf, df, g2, dout_row, dq, stat, dgate);
  if (!colv) return;
  float* dqp = a.dq + (row * a.Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const f32x4 v = dq[dt] * a.scale;
    *reinterpret_cast<f32x4*>(dqp + 16 * dt + 4 * grp) = v;
  }
}

// B operand of the key-side products for a pair of tokens: rows 8 grp + j
// are (token j / 4, head 4 grp + j % 4), column d; from the head-minor copy.
template <class T>
__device__ __forceinline__ Frag<T> pair_rows(const typename T::storage* xa, const typename T::storage* xb);
template <>
__device__ __forceinline__ Frag<BF16> pair_rows<BF16>(const uint16_t* xa, const uint16_t* xb) {
  Frag<BF16> f;
  const uint2 u = *reinterpret_cast<const uint2*>(xa);
  const uint2 w = xb != nullptr ? *reinterpret_cast<const uint2*>(xb) : uint2{0u, 0u};
  f.v = u32x4{u.x, u.y, w.x, w.y};
  return f;
}
template <>
__device__ __forceinline__ Frag<F32> pair_rows<F32>(const float* xa, const float* xb) {
  Frag<F32> f;
  f.lo = *reinterpret_cast<const f32x4*>(xa);
  f.hi = xb != nullptr ? *reinterpret_cast<const f32x4*>(xb) : f32x4{0.f, 0.f, 0.f, 0.f};
  return f;
}

// Key side of branch X: one workgroup per (sequence, group, 64-key chunk,
// piece of the tokens that see it); wave w owns keys [16 w, 16 w + 16) of the
// chunk. The tokens go through LDS kBwdStage at a time, loaded once by the
// whole workgroup (q and dout in both operand layouts, each head's
// log-sum-exp, dout.o and gate), and each wave takes them two at a time (32
// rows of the dK / dV products).
template <class T, int D>
struct BkvStage {
  using S = typename T::storage;
  static constexpr int RS = D + 8;  // padded row of a natural-layout head (16-byte multiple)
  S qn[kBwdStage][16][RS];          // q, [token][head][d]
  S dn[kBwdStage][16][RS];          // dout in the input type
  S qt[kBwdStage][D * 16];          // q, [token][d][head]
  S dt[kBwdStage][D * 16];          // dout, [token][d][head]
  float2 st[kBwdStage][16];         // (log2-domain log-sum-exp, dout . o) of this branch
  float gt[kBwdStage][16];          // this branch's gate
  int tok[kBwdStage];               // token position, -1 past the piece
};

template <class T, int D, int X>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(typename T::storage) == 2 ? 2 : 1))) void
k_bkv(BwdArgs a) {
  using S = typename T::storage;
  constexpr int KS = D / 32, DT = D / 16, TT = kBwdStage;
  extern __shared__ __align__(16) unsigned char bkv_smem[];
  BkvStage<T, D>& sm = *reinterpret_cast<BkvStage<T, D>*>(bkv_smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int nchunk = X == 0 ? a.NcT : a.Nb;
  const int units = a.bkv_units[X];  // units per (sequence, group)
  const int bg = static_cast<int>(blockIdx.x / units), u = static_cast<int>(blockIdx.x % units);
  const int g = bg % a.G, b = bg / a.G;
  // this unit's chunk and token range (window / compressed) or list slice (selected)
  int c, i0, i1;
  const int32_t* list = nullptr;
  if (X == 1) {
    const int32_t* pofs = a.pofs + static_cast<size_t>(bg) * (a.Nb + 1);
    if (u >= pofs[a.Nb]) return;
    int lo = 0, hi = a.Nb - 1;  // the last chunk with pofs <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pofs[mid] <= u) lo = mid;
      else hi = mid - 1;
    }
    c = lo;
    const int32_t* offs = a.offs + static_cast<size_t>(bg) * (a.Nb + 1);
    const int piece = u - pofs[c];
    i0 = offs[c] + piece * kBwdSelPiece;
    i1 = min(offs[c + 1], i0 + kBwdSelPiece);
    list = a.list + static_cast<size_t>(bg) * a.L * a.n;
  } else {
    const int per = units / nchunk;  // pieces per chunk
    c = u / per;
    const int piece = u % per;
    const int tstart = X == 0 ? 64 * 64 * c + 63 : 64 * c;
    const int tend = X == 0 ? a.L : min(a.L, 64 * c + 63 + a.w);
    const int span = (tend - tstart + per - 1) / per;
    i0 = tstart + piece * max(span, 0);
    i1 = min(tend, i0 + max(span, 0));
  }
  if (i0 >= i1) return;  // uniform over the workgroup: no barrier is skipped by part of it
  const float sl2 = a.scale_log2;
  const size_t tile_off = (static_cast<size_t>(bg) * nchunk + c) * 64 * D;
  const S* KA = static_cast<const S*>(X == 0 ? a.kca : a.ka) + tile_off;
  const S* VA = static_cast<const S*>(X == 0 ? a.vca : a.va) + tile_off;
  Frag<T> kb[KS], vb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kb[s] = frag_load<T>(KA + ktile_frag(wave, s, lane, D));
    vb[s] = frag_load<T>(VA + ktile_frag(wave, s, lane, D));
  }
  const int key = 64 * c + 16 * wave + col;  // this lane's key (column of S)
  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int tid = threadIdx.x;
  // Staging, software-pipelined: the next stage's rows are read into
  // registers while this stage is computed, and written to LDS after it. All
  // reads are unconditional, at clamped (token, head) indices, zeroed where
  // not valid, so the loads in flight are the same on every path and the
  // compiler waits only for the stage being written. A stage's tokens come
  // from the selection list (branch 1) one stage ahead of its rows.
  const int e = tid * 8, hh = e / D, d = e % D;
  const bool estage = e < 16 * D;   // 16 x D elements per array and token: all threads at D = 128, half at 64
  const int hc = g * a.Hg + min(hh, a.Hg - 1), hs = g * a.Hg + min(tid & 15, a.Hg - 1);
  auto token_of = [&](int i) -> int {
    if (X == 1) {
      const int v = list[min(i, i1 - 1)];
      return i < i1 ? v : -1;
    }
    return i < i1 ? i : -1;
  };
  Frag<T> rq[TT], rd[TT], rqt[TT], rdt[TT];
  float2 rst[TT];
  float rgt[TT];
  int rtok[TT], ntok[TT];
  auto load_stage = [&](const int (&tok)[TT]) {
#pragma unroll
    for (int uu = 0; uu < TT; ++uu) {
      const int t = tok[uu], tcl = t < 0 ? 0 : t;
      const size_t row = static_cast<size_t>(b) * a.L + tcl;
      const bool tv = t >= 0;
      rq[uu] = frag_load_if<T>(static_cast<const S*>(a.q) + b * a.qs[0] + tcl * a.qs[1] + hc * a.qs[2] + d,
                               estage && tv && hh < a.Hg);
      rd[uu] = frag_load_if<T>(static_cast<const S*>(a.dN) + (row * a.Hq + hc) * D + d, estage && tv && hh < a.Hg);
      rqt[uu] = frag_load_if<T>(static_cast<const S*>(a.qT) + (row * a.G + g) * D * 16 + (estage ? e : 0), estage && tv);
      rdt[uu] = frag_load_if<T>(static_cast<const S*>(a.dT) + (row * a.G + g) * D * 16 + (estage ? e : 0), estage && tv);
      const float2 sv = a.stat[(row * a.Hq + hs) * 3 + X];
      const float gv = to_f32<T>(static_cast<const S*>(a.gates)[b * a.gs[0] + tcl * a.gs[1] + hs * a.gs[2] + X]);
      const bool sok = tv && (tid & 15) < a.Hg;
      rst[uu] = sok ? sv : make_float2(0.f, 0.f);
      rgt[uu] = sok ? gv : 0.f;
      rtok[uu] = t;
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int uu = 0; uu < TT; ++uu) {
      if (estage) {
        frag_store<T>(&sm.qn[uu][hh][d], rq[uu]);
        frag_store<T>(&sm.dn[uu][hh][d], rd[uu]);
        frag_store<T>(&sm.qt[uu][e], rqt[uu]);
        frag_store<T>(&sm.dt[uu][e], rdt[uu]);
      }
      if (tid < 16) {
        sm.st[uu][tid] = rst[uu];
        sm.gt[uu][tid] = rgt[uu];
        if (tid == 0) sm.tok[uu] = rtok[uu];
      }
    }
  };
  {
    int tok[TT];
#pragma unroll
    for (int uu = 0; uu < TT; ++uu) tok[uu] = token_of(i0 + uu);
    load_stage(tok);
#pragma unroll
    for (int uu = 0; uu < TT; ++uu) ntok[uu] = token_of(i0 + TT + uu);
  }
  for (int ib = i0; ib < i1; ib += TT) {
    lds_barrier();  // the previous stage has been read
    store_stage();
    lds_barrier();
    // the next stage's rows (its tokens were read a stage ago), then the
    // tokens of the stage after it
    load_stage(ntok);
#pragma unroll
    for (int uu = 0; uu < TT; ++uu) ntok[uu] = token_of(ib + 2 * TT + uu);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pp = 0; pp < TT; pp += 2) {
      f32x4 P[2], dS[2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int t = sm.tok[pp + uu];
        P[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
        dS[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < 0) continue;
        f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f}, dp4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          mma(s4, frag_load<T>(&sm.qn[pp + uu][col][32 * s + 8 * grp]), kb[s]);
          mma(dp4, frag_load<T>(&sm.dn[pp + uu][col][32 * s + 8 * grp]), vb[s]);
        }
        // lane holds rows (heads) 4 grp + i2 of column `key`
        bool vis;
        if (X == 0) vis = key < a.Nc && 64 * key + 63 <= t;
        else if (X == 1) vis = key <= t;
        else vis = key <= t && key >= t - a.w + 1;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int hh = 4 * grp + i2;
          const float2 stv = sm.st[pp + uu][hh];
          const float p = (vis && hh < a.Hg) ? sm.gt[pp + uu][hh] * fast_exp2(fmaf(s4[i2], sl2, -stv.x)) : 0.f;
          P[uu][i2] = p;
          dS[uu][i2] = p * (dp4[i2] - stv.y);
        }
      }
      const Frag<T> pf = pack_p<T>(P[0], P[1]);
      const Frag<T> sf = pack_p<T>(dS[0], dS[1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int o = (16 * dt + col) * 16 + 4 * grp;
        mma(dv[dt], pf, pair_rows<T>(&sm.dt[pp][o], &sm.dt[pp + 1][o]));
        mma(dk[dt], sf, pair_rows<T>(&sm.qt[pp][o], &sm.qt[pp + 1][o]));
      }
    }
  }
  // lane holds dK / dV of keys 64 c + 16 wave + 4 grp + i2, column 16 dt + col
#pragma unroll
  for (int i2 = 0; i2 < 4; ++i2) {
    const int kk = 64 * c + 16 * wave + 4 * grp + i2;
    float *pk, *pv;
    if (X == 0) {
      if (kk >= a.Nc) continue;
      const size_t o = ((static_cast<size_t>(b) * a.Nc + kk) * a.G + g) * D;
      pk = a.dkc + o;
      pv = a.dvc + o;
    } else {
      if (kk >= a.L) continue;
      const size_t o = ((static_cast<size_t>(b) * a.L + kk) * a.G + g) * D;
      pk = a.dk + o;
      pv = a.dv + o;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      unsafeAtomicAdd(pk + 16 * dt + col, a.scale * dk[dt][i2]);
      unsafeAtomicAdd(pv + 16 * dt + col, dv[dt][i2]);
    }
  }
}

// dk / dv of the tokens of complete blocks += their block mean's gradient / 64.
__global__ __launch_bounds__(256) void k_bfin(BwdArgs a) {
  const size_t per_seq = static_cast<size_t>(a.Nc) * 64 * a.G * a.D;
  const size_t n = static_cast<size_t>(a.B) * per_seq;
  for (size_t e = blockIdx.x * static_cast<size_t>(256) + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * 256) {
    const size_t b = e / per_seq, r = e % per_seq;
    const size_t gd = r % (static_cast<size_t>(a.G) * a.D), t = r / (static_cast<size_t>(a.G) * a.D);
    const size_t src = (b * a.Nc + t / 64) * a.G * a.D + gd;
    const size_t dst = (b * a.L + t) * a.G * a.D + gd;
    a.dk[dst] += a.dkc[src] * (1.0f / 64.0f);
    a.dv[dst] += a.dvc[src] * (1.0f / 64.0f);
  }
}

hipError_t zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 8192));
  hipLaunchKernelGGL(k_bzero, dim3(grid), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

template <class T, class O, int D>
hipError_t launch_backward_t(const BwdArgs& a, hipStream_t st, hipEvent_t* ev) {
  using S = typename T::storage;
  hipError_t e;
  auto rec = [&](int i) { return ev != nullptr ? hipEventRecord(ev[i], st) : hipSuccess; };
  // the key-side kernels' attributes are set before the first launch
  const int lds = static_cast<int>(sizeof(BkvStage<T, D>));
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bkv<T, D, 0>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess ||
      (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bkv<T, D, 1>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess ||
      (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bkv<T, D, 2>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess)
    return e;
  if ((e = rec(0)) != hipSuccess) return e;
  const size_t kv_bytes = static_cast<size_t>(a.B) * a.L * a.G * a.D * sizeof(float);
  const size_t kc_bytes = static_cast<size_t>(a.B) * a.Nc * a.G * a.D * sizeof(float);
  if ((e = zero(a.dk, kv_bytes, st)) != hipSuccess) return e;
  if ((e = zero(a.dv, kv_bytes, st)) != hipSuccess) return e;
  if ((e = zero(a.dkc, kc_bytes, st)) != hipSuccess) return e;
  if ((e = zero(a.dvc, kc_bytes, st)) != hipSuccess) return e;
  if ((e = zero(a.cnt, static_cast<size_t>(a.B) * a.G * a.Nb * sizeof(int32_t), st)) != hipSuccess) return e;
  // block means [B][Nc][G][D] in the input type
  if (a.Nc > 0) {
    const int64_t ks[3] = {a.ks[0], a.ks[2], a.ks[1]}, vs[3] = {a.vs[0], a.vs[2], a.vs[1]};
    const int64_t cs[3] = {static_cast<int64_t>(a.Nc) * a.G * D, D, static_cast<int64_t>(a.G) * D};
    if ((e = launch_compress(a.B, a.G, a.Nc, D, sizeof(S) == 2, a.k, ks, a.v, vs, a.kcm, cs, a.vcm, cs, st)) !=
        hipSuccess)
      return e;
  }
  hipLaunchKernelGGL((k_btile<T, D>), dim3(a.Nb, a.G, a.B), dim3(256), 0, st, static_cast<const S*>(a.k),
                     a.ks[0], a.ks[1], a.ks[2], a.L, a.Nb, static_cast<S*>(a.ka), static_cast<S*>(a.kv));
  hipLaunchKernelGGL((k_btile<T, D>), dim3(a.Nb, a.G, a.B), dim3(256), 0, st, static_cast<const S*>(a.v),
                     a.vs[0], a.vs[1], a.vs[2], a.L, a.Nb, static_cast<S*>(a.va), static_cast<S*>(a.vv));
  if (a.NcT > 0) {
    const int64_t c0 = static_cast<int64_t>(a.Nc) * a.G * D, c1 = static_cast<int64_t>(a.G) * D, c2 = D;
    hipLaunchKernelGGL((k_btile<T, D>), dim3(a.NcT, a.G, a.B), dim3(256), 0, st, static_cast<const S*>(a.kcm),
                       c0, c1, c2, a.Nc, a.NcT, static_cast<S*>(a.kca), static_cast<S*>(a.kcv));
    hipLaunchKernelGGL((k_btile<T, D>), dim3(a.NcT, a.G, a.B), dim3(256), 0, st, static_cast<const S*>(a.vcm),
                       c0, c1, c2, a.Nc, a.NcT, static_cast<S*>(a.vca), static_cast<S*>(a.vcv));
  }
  hipLaunchKernelGGL((k_btrans<T, O, D>), dim3(a.L, a.B), dim3(256), 0, st, a);
  const int64_t rows = static_cast<int64_t>(a.B) * a.L * a.G;
  const unsigned rgrid = static_cast<unsigned>((rows + 255) / 256);
  hipLaunchKernelGGL(k_bsel_count, dim3(rgrid), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_bsel_scan, dim3(a.B * a.G), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_bsel_fill, dim3(rgrid), dim3(256), 0, st, a);
  if ((e = rec(1)) != hipSuccess) return e;
  if (a.lse_slc != nullptr)
    hipLaunchKernelGGL((k_bq<T, O, D, true>), dim3(a.B * a.G * ((a.L + 3) / 4)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_bq<T, O, D, false>), dim3(a.B * a.G * ((a.L + 3) / 4)), dim3(256), 0, st, a);
  if ((e = rec(2)) != hipSuccess) return e;
  if (a.NcT > 0)
    hipLaunchKernelGGL((k_bkv<T, D, 0>), dim3(a.B * a.G * a.bkv_units[0]), dim3(256), lds, st, a);
  hipLaunchKernelGGL((k_bkv<T, D, 1>), dim3(a.B * a.G * a.bkv_units[1]), dim3(256), lds, st, a);
  hipLaunchKernelGGL((k_bkv<T, D, 2>), dim3(a.B * a.G * a.bkv_units[2]), dim3(256), lds, st, a);
  if (a.Nc > 0) {
    const size_t n = static_cast<size_t>(a.B) * a.Nc * 64 * a.G * D;
    hipLaunchKernelGGL(k_bfin, dim3(static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 16384))), dim3(256),
                       0, st, a);
  }
  if ((e = rec(3)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, bool in_bf16, bool out_bf16, hipStream_t st, hipEvent_t* ev) {
  if (in_bf16) {
    if (out_bf16)
      return a.D == 64 ? launch_backward_t<BF16, BF16, 64>(a, st, ev) : launch_backward_t<BF16, BF16, 128>(a, st, ev);
    return a.D == 64 ? launch_backward_t<BF16, F32, 64>(a, st, ev) : launch_backward_t<BF16, F32, 128>(a, st, ev);
  }
  return a.D == 64 ? launch_backward_t<F32, F32, 64>(a, st, ev) : launch_backward_t<F32, F32, 128>(a, st, ev);
}

}  // namespace nsa
