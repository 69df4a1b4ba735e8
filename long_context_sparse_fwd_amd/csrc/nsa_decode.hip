// NSA decode on gfx950: one new query token per sequence against a K/V cache
// and a block-mean cache, measured apart from prefill as the NSA how-to
// (qwbw.cn/news/106443), section 5, advises.
//
// k_dec: one workgroup per (sequence, KV group), 8 waves, one launch. The work
// is HBM-bound -- every key is read once and serves the 16 query heads of its
// group -- so the waves stream it in 32-key half chunks, each wave keeping the
// next one in flight (a register ring) while it computes the current:
//   A  compressed half chunks (block means), dealt round-robin to the waves;
//      the logits are kept (in LDS when they fit) for the block scores;
//   B  the waves' states are merged through LDS into the log-sum-exp and
//      gate_cmp * O_cmp;
//   C  block scores (probabilities summed over the group's heads); then
//      wave 0 selects the own block + top-(n-1) earlier blocks (nsa_topk.h)
//      and lists their usable half blocks while the other waves stream the
//      sliding window, merged into gate_win * O_win;
//   D  the selected half blocks, dealt round-robin to all waves, merged into
//      gate_slc * O_slc;
//   E  the sum of the three gated branches is written to out.
// K rows feed the S^T = K Q^T product straight from the caches. V rows are
// written to LDS row-major (padded so that reads do not conflict) and each
// lane gathers the 8 keys of its V^T operand fragment from there.
#include <hip/hip_ext.h>

#include "nsa_device.h"
#include "nsa_internal.h"
#include "nsa_topk.h"

namespace nsa {

// floats per partial state: m[16], l[16], O[16][D + 4] (rows padded so that
// the 16 heads' rows start in different LDS banks)
__host__ __device__ constexpr int dec_slot_floats(int D) { return 32 + 16 * (D + 4); }

// One wave's registers for 32 keys: K rows as A operands of two key tiles,
// V rows as 8-element vectors (which row and columns a lane holds: v_row,
// v_col).
template <class T, int D>
struct DHalf {
  Frag<T> k[2][D / 32];
  Frag<T> v[D / 16];
};

// V vector i of lane l. bf16: rows come in pairs (2p, 2p + 1) held by the
// same lane, so that the pair can be interleaved into dwords for LDS; fp32:
// row-major order. Each load instruction covers whole rows.
template <class T, int D>
__device__ __forceinline__ int v_row(int lane, int i) {
  constexpr int VPR = D / 8;
  if constexpr (sizeof(typename T::storage) == 2)
    return 2 * (lane / VPR + (64 / VPR) * (i >> 1)) + (i & 1);
  else
    return (lane + 64 * i) / VPR;
}
template <int D>
__device__ __forceinline__ int v_col(int lane) { return (lane % (D / 8)) * 8; }

// A half chunk: keys [key0, key0 + 32) of rows kr / vr, of which those in
// [klo, khi] count (klo <= khi); lrow (or nullptr) receives this lane's
// logits.
template <class T>
struct DItem {
  const typename T::storage* kr;
  const typename T::storage* vr;
  int64_t kst, vst;
  int key0, klo, khi;
  float* lrow;
};

// Rows outside [klo, khi] are loaded from the nearest row inside: their
// logits are masked to -inf, so they get probability 0 and only have to be
// finite. A call reads each cache row once, so the loads are non-temporal.
template <class T, int D>
__device__ __forceinline__ void dhalf_load(DHalf<T, D>& c, const DItem<T>& it, int lane) {
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = min(max(it.key0 + 16 * kt + col, it.klo), it.khi);
    const typename T::storage* p = it.kr + static_cast<int64_t>(key) * it.kst + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) c.k[kt][s] = frag_load_nt<T>(p + 32 * s);
  }
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int key = min(max(it.key0 + v_row<T, D>(lane, i), it.klo), it.khi);
    c.v[i] = frag_load_nt<T>(it.vr + static_cast<int64_t>(key) * it.vst + v_col<D>(lane));
  }
}

// LDS staging of a wave's V half chunk, and the V^T operand fragments read
// back from it. Fragment dt of lane l holds V[kappa(l/16, j)][16 dt + l%16],
// kappa(a, j) = 4a + j (j < 4), 16 + 4a + j - 4 (j >= 4): the keys whose
// probabilities the lane holds in the two S^T tiles (see pack_p). Rows are
// padded by 16 bytes so that the four lane groups of a read hit distinct
// banks.
template <class T, int D>
struct VStage;

// bf16: dword (p, d) holds V[2p][d] (low half) and V[2p + 1][d] (high half),
// so a fragment is four dword reads and needs no repacking.
template <int D>
struct VStage<BF16, D> {
  static constexpr int kRow = D + 8;  // dwords per row pair
  static constexpr size_t kBytes = 16 * kRow * 4;
  __device__ static void put(void* lds, const DHalf<BF16, D>& c, int lane) {
    uint32_t* base = static_cast<uint32_t*>(lds);
#pragma unroll
    for (int q = 0; q < D / 32; ++q) {
      const u32x4 r0 = c.v[2 * q].v, r1 = c.v[2 * q + 1].v;
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = r0[w], y = r1[w];
        const uint32_t e = (x & 0xFFFFu) | (y << 16), o = (x >> 16) | (y & 0xFFFF0000u);
        if (w < 2) {
          lo[2 * w] = e;
          lo[2 * w + 1] = o;
        } else {
          hi[2 * w - 4] = e;
          hi[2 * w - 3] = o;
        }
      }
      uint32_t* dst = base + (v_row<BF16, D>(lane, 2 * q) >> 1) * kRow + v_col<D>(lane);
      *reinterpret_cast<u32x4*>(dst) = lo;
      *reinterpret_cast<u32x4*>(dst + 4) = hi;
    }
  }
  __device__ static Frag<BF16> get(const void* lds, int dt, int lane) {
    const uint32_t* p = static_cast<const uint32_t*>(lds) + 2 * (lane >> 4) * kRow + 16 * dt + (lane & 15);
    Frag<BF16> f;
    f.v = u32x4{p[0], p[kRow], p[8 * kRow], p[9 * kRow]};
    return f;
  }
};

// fp32: row-major.
template <int D>
struct VStage<F32, D> {
  static constexpr int kRow = D + 4;  // floats per row
  static constexpr size_t kBytes = 32 * kRow * 4;
  __device__ static void put(void* lds, const DHalf<F32, D>& c, int lane) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      frag_store<F32>(static_cast<float*>(lds) + v_row<F32, D>(lane, i) * kRow + v_col<D>(lane), c.v[i]);
  }
  __device__ static Frag<F32> get(const void* lds, int dt, int lane) {
    const float* p = static_cast<const float*>(lds) + 4 * (lane >> 4) * kRow + 16 * dt + (lane & 15);
    Frag<F32> f;
    f.lo = f32x4{p[0], p[kRow], p[2 * kRow], p[3 * kRow]};
    f.hi = f32x4{p[16 * kRow], p[17 * kRow], p[18 * kRow], p[19 * kRow]};
    return f;
  }
};

// First half of a step: writes the loaded V rows to this wave's LDS staging
// lv, computes S^T = K Q^T (query fragments qlds[s][lane]) into st and, if
// it.lrow is set, stores this lane's logits. The register buffer c is free
// afterwards.
template <class T, int D>
__device__ __forceinline__ void dhalf_scores(const DHalf<T, D>& c, const DItem<T>& it,
                                             const Frag<T>* qlds, float sl2, void* lv,
                                             f32x4 (&st)[2], int lane) {
  constexpr int KS = D / 32;
  const int grp = lane >> 4;
  VStage<T, D>::put(lv, c, lane);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const Frag<T> qf = qlds[s * 64 + lane];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) mma(st[kt], c.k[kt][s], qf);
  }
  if (it.lrow != nullptr) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = it.key0 + 16 * kt + 4 * grp + i;
        x[i] = (key >= it.klo && key <= it.khi) ? st[kt][i] * sl2 : -INFINITY;
      }
      *reinterpret_cast<f32x4*>(it.lrow + 16 * kt + 4 * grp) = x;
    }
  }
}

// Second half: online-softmax update of (m, l, acc) from st, with the V^T
// fragments read back from the staging one at a time.
template <class T, int D>
__device__ __forceinline__ void dhalf_update(f32x4 (&st)[2], const DItem<T>& it, float sl2, void* lv,
                                             float& m, float& l, f32x4 (&acc)[D / 16], int lane) {
  constexpr int DT = D / 16;
  const int grp = lane >> 4;
  wave_lds_sync();
  const bool full = it.key0 >= it.klo && it.key0 + 31 <= it.khi;
  const Frag<T> pf = full ? online_probs<T, DT, false>(st, it.key0, 0, 0, grp, sl2, m, l, acc)
                          : online_probs<T, DT, true>(st, it.key0, it.klo, it.khi, grp, sl2, m, l, acc);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) mma(acc[dt], VStage<T, D>::get(lv, dt, lane), pf);
  wave_lds_sync();
}

// A wave's half chunks streamed through a ring of RING register buffers.
// A phase is a count N of steps (a multiple of RING, at least RING) and
// item(k), the k-th step's half chunk; steps past the wave's real items are
// empty items (an empty key range over rows the wave has just read, so the
// reload hits the caches). All rounds but the last refill each buffer as
// soon as it is consumed, unconditionally: the number of loads in flight is
// then the same on every path, so each step waits only for its own buffer.
// The last round refills nothing, so a phase ends with no loads in flight;
// the next phase's ring is primed (prime()) where it can overlap other work.
template <class T, int D, int RING>
struct DStream {
  DHalf<T, D> ring[RING];
  template <class Item>
  __device__ __forceinline__ void prime(Item item, int lane) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      dhalf_load<T, D>(ring[r], item(r), lane);
      __builtin_amdgcn_sched_barrier(0);  // buffers in order
    }
  }
  // One round: steps k0 .. k0 + RING - 1. scores(c, it, st) consumes buffer
  // c into st; update(st, it) finishes the step. With REFILL, each buffer is
  // refilled with step k0 + r + RING between the two, so its loads are in
  // flight during the softmax and the P.V product.
  template <bool REFILL, class Item, class Scores, class Update>
  __device__ __forceinline__ void round(int k0, Item item, Scores scores, Update update, int lane) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const DItem<T> it = item(k0 + r);
      f32x4 st[2];
      scores(ring[r], it, st);
      if constexpr (REFILL) {
        __builtin_amdgcn_sched_barrier(0);
        dhalf_load<T, D>(ring[r], item(k0 + r + RING), lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      update(st, it);
    }
  }
  template <class Item, class Scores, class Update>
  __device__ __forceinline__ void run(int N, Item item, Scores scores, Update update, int lane) {
#pragma unroll 1
    for (int k0 = 0; k0 < N - RING; k0 += RING) round<true>(k0, item, scores, update, lane);
    round<false>(N - RING, item, scores, update, lane);
  }
};

// Steps of a phase whose wave holds n real items: n rounded up to a whole
// number of rounds, at least one round.
template <int RING>
__device__ __forceinline__ int phase_steps(int n) {
  return n > RING ? (n + RING - 1) / RING * RING : RING;
}

// The same rows, as an empty key range (nothing is added; no logits).
template <class T>
__device__ __forceinline__ DItem<T> empty_item(DItem<T> it) {
  it.klo = it.khi + 1;
  it.lrow = nullptr;
  return it;
}

// Stores a wave's partial state (m per column, l summed over the column's
// lanes, O^T accumulators) as m[16], l[16], O[16][D + 4] at dst.
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
    *reinterpret_cast<f32x4*>(dst + 32 + col * (D + 4) + 16 * dt + 4 * grp) = acc[dt];
}

// Merge factors of head h over CNT partial states (stride SF floats, one
// thread per head): M = max_w m_w, L = sum_w l_w 2^(m_w - M), and
// fac[w][h] = 2^(m_w - M) gate / L (0 when L = 0), so that the merged, gated
// output element e of head h is sum_w O_w[e] fac[w][h].
template <int CNT>
__device__ __forceinline__ void merge_factors(const float* p, int SF, int h, float gate, float* fac, float& M,
                                              float& L) {
  float mw[CNT];
  M = kNegBig;
#pragma unroll
  for (int w = 0; w < CNT; ++w) {
    mw[w] = p[w * SF + h];
    M = fmaxf(M, mw[w]);
  }
  L = 0.f;
#pragma unroll
  for (int w = 0; w < CNT; ++w) {
    mw[w] = fast_exp2(mw[w] - M);
    L += p[w * SF + 16 + h] * mw[w];
  }
  const float r = L > 0.f ? gate / L : 0.f;
#pragma unroll
  for (int w = 0; w < CNT; ++w) fac[w * 16 + h] = mw[w] * r;
}

// Elements e .. e + 3 (e = h D + d, d a multiple of 4; head h) of the
// merged, gated output.
template <int CNT, int D>
__device__ __forceinline__ f32x4 merge_out4(const float* p, const float* fac, int SF, int e) {
  const int h = e / D, off = 32 + e + 4 * h;  // O[h][d] of a partial state
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < CNT; ++w) o += *reinterpret_cast<const f32x4*>(p + w * SF + off) * fac[w * 16 + h];
  return o;
}

template <int D>
__device__ __forceinline__ void reset_state(float& m, float& l, f32x4 (&acc)[D / 16]) {
  m = kNegBig;
  l = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}


// Block scores sc[j], j < own: the compressed-branch probabilities of block
// j summed over the group's heads, from the logits lg[h][j] (row stride ld)
// and each head's log-sum-exp hs[4 h + 2]. Rows of heads h >= Hg hold finite
// logits and have log-sum-exp +inf, so they add exact zeros.
template <class P>
__device__ __forceinline__ void block_scores(P lg, int ld, int own, const float* hs, float* sc, int tid,
                                             int nt) {
  float lse[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) lse[h] = hs[4 * h + 2];
  for (int j = tid; j < own; j += nt) {
    float x[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) x[h] = lg[h * ld + j];
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < 16; ++h) s += fast_exp2(x[h] - lse[h]);
    sc[j] = s;
  }
}

// Per-wave partial states live in the wave's own V staging (stride PS
// floats), so a wave can store its state without waiting for the others.
template <class T, int D>
__host__ __device__ constexpr int dec_part_stride() {
  return static_cast<int>(VStage<T, D>::kBytes / sizeof(float));
}

// Waits until the LDS counter *flag equals v (set by other waves of the
// workgroup with release stores or adds).
__device__ __forceinline__ void lds_wait_eq(int* flag, int v) {
  while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != v) __builtin_amdgcn_s_sleep(1);
}

// Merges the per-wave states (m, l, acc) of one branch through LDS and adds
// gate[h] * O of the branch to res[16][D] (LDS). Thread tid owns the
// elements 4 tid .. 4 tid + 3 of res in every merge and in the output
// store, so res needs no barrier of its own. Ends with a workgroup barrier, so the V staging may be
// written again afterwards.
template <class T, int D, int NWV>
__device__ __forceinline__ void merge_into(float* parts, float m, float l, const f32x4 (&acc)[D / 16],
                                           const float* gate, float* fac, float* res, int tid, int lane) {
  constexpr int PS = dec_part_stride<T, D>();
  store_partial<D>(parts + (tid >> 6) * PS, m, l, acc, lane);
  lds_barrier();
  if (tid < 16) {
    float M, L;
    merge_factors<NWV>(parts, PS, tid, gate[tid], fac, M, L);
  }
  lds_barrier();
  if (4 * tid < 16 * D)
    *reinterpret_cast<f32x4*>(res + 4 * tid) += merge_out4<NWV, D>(parts, fac, PS, 4 * tid);
  lds_barrier();
}

// General geometry: the selection-block scores from the compressed-block
// scores, in place (sc[0 .. own) on return): the compressed-attention mass on
// each selection block's tokens, every compressed block's probability spread
// evenly over its cl tokens. Selection block j reads compressed blocks i >= j
// only (cd <= cl <= ls), so rounds of 64 blocks can overwrite the scores they
// have consumed. One wave, uniform arguments.
__device__ inline void dec_selection_scores(const DecodeArgs& a, float* sc, int own, int nv, int lane) {
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

// Gate layer of the decode: gates32[b][h][c] = sigmoid(q[b][h] . gate_w[h][:, c]
// + gate_b[h][c]) in fp32, one thread per (sequence, head). The gates of the
// three branches are learned (NSA how-to, qwbw.cn/news/106443, section 3,
// gate_type learned); here a one-layer map of the head's query, as in the
// prefill.
template <class T, int D>
__global__ __launch_bounds__(256) void k_dgate(DecodeArgs a) {
  using S = typename T::storage;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.B * a.Hq) return;
  const int b = e / a.Hq, h = e % a.Hq;
  const S* q = static_cast<const S*>(a.q) + b * a.qs[0] + h * a.qs[1];
  const S* w = static_cast<const S*>(a.gate_w) + static_cast<int64_t>(h) * D * 3;
  const S* bg = static_cast<const S*>(a.gate_b) + 3 * h;
  float z0 = to_f32<T>(bg[0]), z1 = to_f32<T>(bg[1]), z2 = to_f32<T>(bg[2]);
  for (int d = 0; d < D; ++d) {
    const float x = to_f32<T>(q[d]);
    z0 = fmaf(x, to_f32<T>(w[3 * d]), z0);
    z1 = fmaf(x, to_f32<T>(w[3 * d + 1]), z1);
    z2 = fmaf(x, to_f32<T>(w[3 * d + 2]), z2);
  }
  float* o = a.gates32 + static_cast<int64_t>(e) * 3;
  o[0] = 1.0f / (1.0f + fast_exp2(-z0 * kLog2e));
  o[1] = 1.0f / (1.0f + fast_exp2(-z1 * kLog2e));
  o[2] = 1.0f / (1.0f + fast_exp2(-z2 * kLog2e));
}

constexpr int kDecWaves = 8;

template <class T, int D>
__host__ __device__ constexpr size_t dec_big_bytes() {
  static_assert(dec_part_stride<T, D>() >= dec_slot_floats(D), "a partial state must fit a wave's V staging");
  return static_cast<size_t>(kDecWaves) * VStage<T, D>::kBytes;
}

// LGL: the compressed logits stay in LDS. PARK (requires LGL): the logits
// region, free once the block scores are done, holds the 7 window states.
// GEN: the general geometry (stride, selection blocks of ls tokens, gates
// from the gate layer); without it the plain one (blocks of 64, stride 64).
template <class T, class O, int D, int RING, bool LGL, bool PARK, bool GEN>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dec(DecodeArgs a) {
  using S = typename T::storage;
  using SO = typename O::storage;
  constexpr int NWV = kDecWaves, NT = 64 * NWV, SF = dec_slot_floats(D), DT = D / 16;
  constexpr int PS = dec_part_stride<T, D>();
  extern __shared__ __align__(16) unsigned char smem[];
  float* parts = reinterpret_cast<float*>(smem);  // wave w's state in its V staging, at w * PS
  Frag<T>* qlds = reinterpret_cast<Frag<T>*>(smem + dec_big_bytes<T, D>());  // [D/32][64]
  float* res = reinterpret_cast<float*>(qlds + D / 32 * 64);                  // [16][D] output
  float* sc = res + 16 * D;
  uint64_t* surv = reinterpret_cast<uint64_t*>(sc + a.NmaxPad);
  int* selb = reinterpret_cast<int*>(surv + kSurvCap);
  int* selo = selb + 64;
  int* hl = selo + 64;                            // usable selected half blocks: 2 j + half
  int* nhl = hl + 128;                            // their count
  int* hl_ready = nhl + 1;                        // set by wave 0 once hl and nhl are written
  int* parked = nhl + 2;                          // window states parked so far
  float* hs = reinterpret_cast<float*>(nhl + 4);  // per head: 4 floats
  float* gts = hs + 64;                           // [3][16] gates
  float* fac = gts + 48;                          // [NWV][16] merge factors
  float* facw = fac + 16 * NWV;                   // [NWV - 1][16] merge factors of the parked window states
  float* lg_lds = facw + 16 * NWV;                // [16][NmaxPad + 4] logits, if LGL

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: phase counts and bases stay scalar
  const int bg = blockIdx.x, b = bg / a.G, g = bg % a.G;
  const int s_raw = a.seqlens[b];
  int32_t* idxo = a.idx + static_cast<int64_t>(bg) * a.n;
  SO* OUT = static_cast<SO*>(a.out) + b * a.os[0];
  if (s_raw < 1 || s_raw > a.Lmax) {  // invalid length: nothing of this sequence is read
    for (int e = tid; e < a.Hg * D; e += NT) OUT[(g * a.Hg + e / D) * a.os[1] + e % D] = from_f32<O>(0.f);
    if (!a.inject && tid < a.n) idxo[tid] = -1;
    return;
  }
  // visible compressed blocks and the own selection block
  const int t = s_raw - 1;
  const int nvis = GEN ? (s_raw >= a.cl ? (s_raw - a.cl) / a.cd + 1 : 0) : s_raw >> 6;
  const int own = GEN ? t / a.ls : t >> 6;
  const int wlo = max(0, s_raw - a.w);
  const float sl2 = a.scale_log2;
  void* lv = smem + wave * VStage<T, D>::kBytes;

  const S* KCr = static_cast<const S*>(a.kccache) + b * a.kcs[0] + g * a.kcs[1];
  const S* VCr = static_cast<const S*>(a.vccache) + b * a.vcs[0] + g * a.vcs[1];
  const S* Kr = static_cast<const S*>(a.kcache) + b * a.ks[0] + g * a.ks[1];
  const S* Vr = static_cast<const S*>(a.vcache) + b * a.vs[0] + g * a.vs[1];
  // compressed logits, row h = head: in LDS when they fit, else in the workspace
  float* lg = LGL ? lg_lds : a.logits + static_cast<int64_t>(bg) * 16 * a.NmaxPad;
  // row stride of the logits: in LDS padded so that the heads' rows start in
  // different banks
  const int ld = LGL ? a.NmaxPad + 4 : a.NmaxPad;

  float m, l;
  f32x4 acc[DT];
  auto scores = [&](const DHalf<T, D>& c, const DItem<T>& it, f32x4 (&st)[2]) {
    dhalf_scores<T, D>(c, it, qlds, sl2, lv, st, lane);
  };
  auto update = [&](f32x4 (&st)[2], const DItem<T>& it) { dhalf_update<T, D>(st, it, sl2, lv, m, l, acc, lane); };

  // The three phases' items for this wave: the compressed half chunks
  // wave, wave + 8, ...; the window's (wave - 1), (wave - 1) + 7, ... for
  // waves 1..7; the selected half blocks wave, wave + 8, ... Past a wave's
  // real items the steps are empty items; `none` (row 0 of the cache, always
  // present) stands in when a wave has no real item in a phase.
  const DItem<T> none{Kr, Vr, a.ks[2], a.vs[2], 0, 1, 0, nullptr};
  const int ncmp = (nvis + 31) >> 5;
  const int nA = wave < ncmp ? (ncmp - 1 - wave) / NWV + 1 : 0;
  float* lrow = a.inject ? nullptr : lg + col * ld;
  auto a_real = [&](int q) {
    return DItem<T>{KCr, VCr, a.kcs[2], a.vcs[2], 32 * q, 0, nvis - 1, lrow != nullptr ? lrow + 32 * q : nullptr};
  };
  auto a_item = [&](int k) {
    return k < nA ? a_real(wave + NWV * k) : (nA > 0 ? empty_item(a_real(wave + NWV * (nA - 1))) : none);
  };
  const int nwin = (t - wlo + 32) >> 5, wq = wave - 1;
  const int nW = (wave > 0 && wq < nwin) ? (nwin - 1 - wq) / (NWV - 1) + 1 : 0;
  auto w_real = [&](int q) { return DItem<T>{Kr, Vr, a.ks[2], a.vs[2], wlo + 32 * q, wlo, t, nullptr}; };
  auto w_item = [&](int k) {
    return k < nW ? w_real(wq + (NWV - 1) * k) : (nW > 0 ? empty_item(w_real(wq + (NWV - 1) * (nW - 1))) : none);
  };
  int nD = -1;  // known once wave 0 has published the selected half blocks
  auto d_real = [&](int q) {
    const int u = hl[q];   // the half block of keys [32 u, 32 u + 32)
    if constexpr (GEN) return DItem<T>{Kr, Vr, a.ks[2], a.vs[2], 32 * u, 32 * u, t, nullptr};
    const int j = u >> 1;
    return DItem<T>{Kr, Vr, a.ks[2], a.vs[2], 64 * j + 32 * (u & 1), 64 * j, t, nullptr};
  };
  auto d_item = [&](int k) {
    return k < nD ? d_real(wave + NWV * k) : (nD > 0 ? empty_item(d_real(wave + NWV * (nD - 1))) : none);
  };
  auto d_wait = [&]() {
    if (nD < 0) {
      lds_wait_eq(hl_ready, 1);  // wave 0 always publishes the list
      const int nh = *nhl;
      nD = wave < nh ? (nh - 1 - wave) / NWV + 1 : 0;
    }
  };
  DStream<T, D, RING> ds;

  // ---- A: compressed half chunks. Every wave reads the query fragments
  //      (lane l: head l % 16) and the gates of the group's heads first, at
  //      clamped indices and outside any branch, so nothing waits for them
  //      here; then it issues its first loads, whose latency overlaps the
  //      staging of the query by wave 0 (loads return in order, so waiting
  //      for the query does not wait for them).
  Frag<T> qv[D / 32];
  float gv;
  {
    const int hq = col < a.Hg ? col : 0;
    const S* Q = static_cast<const S*>(a.q) + b * a.qs[0] + (g * a.Hg + hq) * a.qs[1] + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qv[s] = frag_load_if<T>(Q + 32 * s, col < a.Hg);
    const int h = lane & 15, i = min(lane >> 4, 2);
    float gg;
    if constexpr (GEN) {
      if (a.gates32 != nullptr)
        gg = a.gates32[(static_cast<int64_t>(b) * a.Hq + g * a.Hg + min(h, a.Hg - 1)) * 3 + i];
      else
        gg = to_f32<T>(static_cast<const S*>(a.gates)[b * a.gs[0] + (g * a.Hg + min(h, a.Hg - 1)) * a.gs[1] + i]);
    } else {
      gg = to_f32<T>(static_cast<const S*>(a.gates)[b * a.gs[0] + (g * a.Hg + min(h, a.Hg - 1)) * a.gs[1] + i]);
    }
    gv = lane < 48 && h < a.Hg ? gg : 0.f;
  }
  ds.prime(a_item, lane);
  if (tid == 0) {
    *hl_ready = 0;
    *parked = 0;
  }
  if (wave == 0) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qlds[s * 64 + lane] = qv[s];
    if (lane < 48) gts[16 * (lane >> 4) + (lane & 15)] = gv;
  }
  lds_barrier();
  reset_state<D>(m, l, acc);
  ds.run(phase_steps<RING>(nA), a_item, scores, update, lane);
  l = col_sum4(l);

  // ---- B: merge into the log-sum-exp and gate_cmp * O_cmp
  store_partial<D>(parts + wave * PS, m, l, acc, lane);
  // partial states and logits written (the logits to global memory when they
  // are not in LDS)
  if constexpr (LGL)
    lds_barrier();
  else
    __syncthreads();
  if (tid < 16) {
    float M, L;
    merge_factors<NWV>(parts, PS, tid, gts[tid], fac, M, L);
    hs[4 * tid + 2] = (nvis > 0 && tid < a.Hg) ? M + fast_log2(L) : INFINITY;
  }
  lds_barrier();
  if (4 * tid < 16 * D) *reinterpret_cast<f32x4*>(res + 4 * tid) = merge_out4<NWV, D>(parts, fac, PS, 4 * tid);

  // ---- C: block scores
  if (!a.inject) {
    block_scores(lg, ld, GEN ? nvis : own, hs, sc, tid, NT);
  }
  lds_barrier();  // sc written; parts read, so the V staging is free again
  // waves 1..7 issue their first window loads; their streams cover the top-k
  if (wave > 0) ds.prime(w_item, lane);

  // ---- C': wave 0 selects and lists the usable half blocks while the other
  //      waves stream the sliding window
  if (wave == 0) {
    if (!a.inject) {
      if constexpr (GEN) dec_selection_scores(a, sc, own, nvis, lane);
      topk_wave(sc, own, a.n, selo, surv, selb, lane);
      wave_lds_sync();
      if (lane < a.n) idxo[lane] = selo[lane];
    } else if (lane < a.n) {
      selo[lane] = idxo[lane];
    }
    wave_lds_sync();
    const int j = lane < a.n ? selo[lane] : -1;
    // the selection is a set of blocks: a repeated injected entry adds nothing
    // (a computed selection has no repeats)
    bool rep = false;
    if (a.inject)
      for (int k = 0; k < a.n; ++k) rep |= k < lane && __builtin_amdgcn_readlane(j, k) == j;
    const bool h0 = j >= 0 && j <= own && !rep;
    // The own block goes first: its keys end the sliding window, which the
    // other waves have just streamed, so its reads still hit L2 (listed last
    // it was read again from HBM, ~8 MB per call at d64k).
    const bool isown = h0 && j == own;
    if constexpr (GEN) {
      // block j's half blocks j * hpb .. that start at or before t
      const int hpb = a.ls >> 5;
      const int cnt = h0 ? min(hpb, (t >> 5) - j * hpb + 1) : 0;
      const int other = isown ? 0 : cnt;
      int incl = other;   // inclusive prefix over the lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const uint64_t bo = __ballot(isown);
      const int nown = bo != 0 ? __shfl(cnt, static_cast<int>(__builtin_ctzll(bo)), 64) : 0;
      const int pos = isown ? 0 : nown + incl - other;
      for (int i = 0; i < cnt; ++i) hl[pos + i] = j * hpb + i;
      if (lane == 63) *nhl = nown + incl;
    } else {
      const bool h1 = h0 && 64 * j + 32 <= t;
      const uint64_t b0 = __ballot(h0), b1 = __ballot(h1);
      const uint64_t below = (uint64_t{1} << lane) - 1;
      const uint64_t bo = __ballot(isown);
      const int nown = bo != 0 ? 1 + ((__ballot(isown && h1) != 0) ? 1 : 0) : 0;
      const uint64_t rest = below & ~bo;
      const int pos = isown ? 0 : nown + __popcll(b0 & rest) + __popcll(b1 & rest);
      if (h0) hl[pos] = 2 * j;
      if (h1) hl[pos + 1] = 2 * j + 1;
      if (lane == 0) *nhl = __popcll(b0) + __popcll(b1);
    }
    wave_lds_sync();  // every lane's hl entries before the flag
    if (lane == 0) __hip_atomic_store(hl_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // The window is streamed by waves 1..7. When the logits region (free once
  // the scores are done) can hold the 7 window states, each wave parks its
  // state there and goes on to the selected blocks as soon as wave 0 has
  // published them, and the window is merged at the end. Otherwise the
  // window is merged before the selected blocks.
  reset_state<D>(m, l, acc);
  if (wave > 0) ds.run(phase_steps<RING>(nW), w_item, scores, update, lane);
  l = col_sum4(l);
  if constexpr (PARK) {
    if (wave > 0) {
      store_partial<D>(lg_lds + (wave - 1) * SF, m, l, acc, lane);
      wave_lds_sync();
      if (lane == 0) __hip_atomic_fetch_add(parked, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  } else {
    merge_into<T, D, NWV>(parts, m, l, acc, gts + 32, fac, res, tid, lane);
  }

  // ---- D: selected half blocks
  d_wait();
  ds.prime(d_item, lane);
  reset_state<D>(m, l, acc);
  ds.run(phase_steps<RING>(nD), d_item, scores, update, lane);
  l = col_sum4(l);
  // The window states were parked before the selected blocks; wave 0, whose
  // share of them ends first, takes their merge factors while the other
  // waves finish.
  if constexpr (PARK) {
    if (wave == 0) {
      lds_wait_eq(parked, NWV - 1);
      if (lane < 16) {
        float M, L;
        merge_factors<NWV - 1>(lg_lds, SF, lane, gts[32 + lane], facw, M, L);
      }
    }
  }
  // ---- merge of the selected-block states (and of the parked window states)
  store_partial<D>(parts + wave * PS, m, l, acc, lane);
  lds_barrier();
  if (tid < 16) {
    float M, L;
    merge_factors<NWV>(parts, PS, tid, gts[16 + tid], fac, M, L);
  }
  lds_barrier();
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  if (4 * tid < 16 * D) {
    o = *reinterpret_cast<const f32x4*>(res + 4 * tid) + merge_out4<NWV, D>(parts, fac, PS, 4 * tid);
    if constexpr (PARK) o += merge_out4<NWV - 1, D>(lg_lds, facw, SF, 4 * tid);
  }

  // ---- E: out = gate_cmp O_cmp + gate_slc O_slc + gate_win O_win
  if (4 * tid < a.Hg * D) {
    SO* o4 = OUT + (g * a.Hg + 4 * tid / D) * a.os[1] + 4 * tid % D;
#pragma unroll
    for (int i = 0; i < 4; ++i) o4[i] = from_f32<O>(o[i]);
  }
}

size_t dec_lds_bytes(int NmaxPad, int D, bool bf16, bool logits_lds) {
  const size_t big = bf16 ? (D == 64 ? dec_big_bytes<BF16, 64>() : dec_big_bytes<BF16, 128>())
                          : (D == 64 ? dec_big_bytes<F32, 64>() : dec_big_bytes<F32, 128>());
  const size_t qbytes = (bf16 ? 16 : 32) * static_cast<size_t>(D / 32) * 64;
  return big + qbytes + 16 * static_cast<size_t>(D) * sizeof(float) + NmaxPad * sizeof(float) +
         kSurvCap * sizeof(uint64_t) + (64 + 64 + 128 + 4) * sizeof(int) + (64 + 48 + 32 * kDecWaves) * sizeof(float) +
         (logits_lds ? 16 * static_cast<size_t>(NmaxPad + 4) * sizeof(float) : 0);
}

template <class T, class O, int D, bool LGL, bool PARK, bool GEN>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st, hipEvent_t* ev) {
  constexpr bool kBf16 = sizeof(typename T::storage) == 2;
  constexpr int RING = kBf16 ? 2 : 1;
  const size_t lds = dec_lds_bytes(a.NmaxPad, D, kBf16, LGL);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec<T, O, D, RING, LGL, PARK, GEN>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  if (GEN && a.gates32 != nullptr) {
    hipLaunchKernelGGL((k_dgate<T, D>), dim3((a.B * a.Hq + 255) / 256), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev != nullptr) {
    // the dispatch itself records the events at the kernel's start and end,
    // so the interval is the kernel's own duration (no launch latency)
    void* args[] = {const_cast<DecodeArgs*>(&a)};
    e = hipExtLaunchKernel(reinterpret_cast<const void*>(&k_dec<T, O, D, RING, LGL, PARK, GEN>), dim3(a.B * a.G),
                           dim3(64 * kDecWaves), args, lds, st, ev[0], ev[1], 0);
    return e != hipSuccess ? e : hipGetLastError();
  }
  hipLaunchKernelGGL((k_dec<T, O, D, RING, LGL, PARK, GEN>), dim3(a.B * a.G), dim3(64 * kDecWaves), lds, st, a);
  return hipGetLastError();
}

template <class T, class O, int D, bool GEN>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t st, hipEvent_t* ev) {
  if (!a.logits_lds) return launch_decode_t<T, O, D, false, false, GEN>(a, st, ev);
  const bool park =
      16 * static_cast<size_t>(a.NmaxPad + 4) >= (kDecWaves - 1) * static_cast<size_t>(dec_slot_floats(D));
  return park ? launch_decode_t<T, O, D, true, true, GEN>(a, st, ev)
              : launch_decode_t<T, O, D, true, false, GEN>(a, st, ev);
}

template <class T, class O, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st, hipEvent_t* ev) {
  return a.gen ? launch_decode_g<T, O, D, true>(a, st, ev) : launch_decode_g<T, O, D, false>(a, st, ev);
}

hipError_t launch_decode(const DecodeArgs& a, bool in_bf16, bool out_bf16, hipStream_t st,
                         hipEvent_t* ev) {
  if (in_bf16) {
    if (out_bf16)
      return a.D == 64 ? launch_decode_d<BF16, BF16, 64>(a, st, ev)
                       : launch_decode_d<BF16, BF16, 128>(a, st, ev);
    return a.D == 64 ? launch_decode_d<BF16, F32, 64>(a, st, ev)
                     : launch_decode_d<BF16, F32, 128>(a, st, ev);
  }
  return a.D == 64 ? launch_decode_d<F32, F32, 64>(a, st, ev) : launch_decode_d<F32, F32, 128>(a, st, ev);
}

}  // namespace nsa
