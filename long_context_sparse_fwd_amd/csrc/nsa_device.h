// Device helpers shared by the libnsa kernels (gfx950 / CDNA4, wave64).
//
// Matrix products use v_mfma_f32_16x16x32_bf16 for bf16 operands and eight
// v_mfma_f32_16x16x4_f32 for fp32 operands. Both consume the same "fragment":
// lane l of a wave holds 8 consecutive k-values of one operand row or column,
//   A (16 x 32):  lane l holds A[m = l % 16][k = 8*(l/16) + j], j = 0..7
//   B (32 x 16):  lane l holds B[k = 8*(l/16) + j][n = l % 16]
//   C (16 x 16):  lane l holds C[m = 4*(l/16) + i][n = l % 16], i = 0..3
// For fp32 the j-th of the eight 16x16x4 products takes value j of both
// operands; it contracts over k-slots {8a + j}, so the eight together cover
// all 32 k-slots, which is all a contraction needs.
//
// Attention is computed transposed (S^T = K Q^T, O^T = V^T P^T) so that the
// C layout of S^T (keys along registers, queries along lanes) is, after a
// fixed permutation of the 32 keys of one k-step, already the B operand of the
// P.V product. The permutation is baked into the stored V tiles (see
// vtile_off), so no data moves between the two products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element type tags.
struct BF16 {
  using storage = uint16_t;
};
struct F32 {
  using storage = float;
};

template <class T>
struct Frag;
template <>
struct Frag<BF16> {
  u32x4 v;
};
template <>
struct Frag<F32> {
  f32x4 lo, hi;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Two floats -> two bf16 (round to nearest even) packed low/high in 32 bits:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

template <class T>
__device__ __forceinline__ float to_f32(typename T::storage x);
template <>
__device__ __forceinline__ float to_f32<BF16>(uint16_t x) {
  return bf16_to_f32(x);
}
template <>
__device__ __forceinline__ float to_f32<F32>(float x) {
  return x;
}

template <class T>
__device__ __forceinline__ typename T::storage from_f32(float x);
template <>
__device__ __forceinline__ uint16_t from_f32<BF16>(float x) {
  return static_cast<uint16_t>(f32_to_bf16_bits(x));
}
template <>
__device__ __forceinline__ float from_f32<F32>(float x) {
  return x;
}

// A fragment of ones (every one of the 8 elements is 1.0).
template <class T>
__device__ __forceinline__ Frag<T> frag_ones();
template <>
__device__ __forceinline__ Frag<BF16> frag_ones<BF16>() {
  Frag<BF16> f;
  f.v = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  return f;
}
template <>
__device__ __forceinline__ Frag<F32> frag_ones<F32>() {
  Frag<F32> f;
  f.lo = f32x4{1.f, 1.f, 1.f, 1.f};
  f.hi = f.lo;
  return f;
}

template <class T>
__device__ __forceinline__ Frag<T> frag_zero();
template <>
__device__ __forceinline__ Frag<BF16> frag_zero<BF16>() {
  Frag<BF16> f;
  f.v = u32x4{0u, 0u, 0u, 0u};
  return f;
}
template <>
__device__ __forceinline__ Frag<F32> frag_zero<F32>() {
  Frag<F32> f;
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
  return f;
}

// 8 consecutive elements (16 B for bf16, 32 B for fp32); p must be aligned to that.
template <class T>
__device__ __forceinline__ Frag<T> frag_load(const typename T::storage* p);
template <>
__device__ __forceinline__ Frag<BF16> frag_load<BF16>(const uint16_t* p) {
  Frag<BF16> f;
  f.v = *reinterpret_cast<const u32x4*>(p);
  return f;
}
template <>
__device__ __forceinline__ Frag<F32> frag_load<F32>(const float* p) {
  Frag<F32> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}

// frag_load for rows a kernel reads once (a decode step's K/V rows):
// non-temporal loads, which stream from HBM about 10 % faster than cached
// ones (6.4-6.5 against 5.8-6.0 TB/s for 320 MiB after a cache flush).
template <class T>
__device__ __forceinline__ Frag<T> frag_load_nt(const typename T::storage* p);
template <>
__device__ __forceinline__ Frag<BF16> frag_load_nt<BF16>(const uint16_t* p) {
  Frag<BF16> f;
  f.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return f;
}
template <>
__device__ __forceinline__ Frag<F32> frag_load_nt<F32>(const float* p) {
  Frag<F32> f;
  f.lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  f.hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  return f;
}

template <class T>
__device__ __forceinline__ void frag_store(typename T::storage* p, const Frag<T>& f);
template <>
__device__ __forceinline__ void frag_store<BF16>(uint16_t* p, const Frag<BF16>& f) {
  *reinterpret_cast<u32x4*>(p) = f.v;
}
template <>
__device__ __forceinline__ void frag_store<F32>(float* p, const Frag<F32>& f) {
  *reinterpret_cast<f32x4*>(p) = f.lo;
  *reinterpret_cast<f32x4*>(p + 4) = f.hi;
}

// c += A.B for one 16x16x32 step.
__device__ __forceinline__ void mma(f32x4& c, const Frag<BF16>& a, const Frag<BF16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                               __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<F32>& a, const Frag<F32>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
}

// Two C-layout tiles of probabilities (keys 0..15 and 16..31 of one k-step)
// -> the B operand of the P.V product, in the permuted key order of vtile_off.
template <class T>
__device__ __forceinline__ Frag<T> pack_p(const f32x4& a, const f32x4& b);
template <>
__device__ __forceinline__ Frag<BF16> pack_p<BF16>(const f32x4& a, const f32x4& b) {
  Frag<BF16> f;
  f.v.x = pack_bf16x2(a.x, a.y);
  f.v.y = pack_bf16x2(a.z, a.w);
  f.v.z = pack_bf16x2(b.x, b.y);
  f.v.w = pack_bf16x2(b.z, b.w);
  return f;
}
template <>
__device__ __forceinline__ Frag<F32> pack_p<F32>(const f32x4& a, const f32x4& b) {
  Frag<F32> f;
  f.lo = a;
  f.hi = b;
  return f;
}

// ---------------------------------------------------------------- tile layouts
//
// A 64-key chunk of K (64 x D) is stored "fragment-major": the A-operand
// fragment (key-tile kt, k-step s) of lane l is 8 contiguous elements at
// ((kt * D/32 + s) * 64 + l) * 8, holding K[16 kt + l%16][32 s + 8 (l/16) + j].
// One fragment load of a wave is therefore 64 x 8 contiguous elements.
__host__ __device__ __forceinline__ int ktile_off(int r, int d, int D) {
  const int kt = r >> 4, s = d >> 5;
  const int lane = (r & 15) + 16 * ((d & 31) >> 3);
  return ((kt * (D >> 5) + s) * 64 + lane) * 8 + (d & 7);
}
__host__ __device__ __forceinline__ int ktile_frag(int kt, int s, int lane, int D) {
  return ((kt * (D >> 5) + s) * 64 + lane) * 8;
}

// A 64-key chunk of V^T (D x 64): the A-operand fragment (d-tile dt, k-step s)
// of lane l is 8 contiguous elements at ((dt * 2 + s) * 64 + l) * 8 holding
// V[32 s + kappa(l/16, j)][16 dt + l%16], kappa(a, j) = 4a + j for j < 4 and
// 16 + 4a + (j - 4) otherwise: exactly the keys whose probabilities lane l
// holds in the C layout of the two S^T tiles of that k-step.
__host__ __device__ __forceinline__ int vtile_off(int r, int d) {
  const int s = r >> 5, rr = r & 31;
  const int half = rr >> 4, a = (rr & 15) >> 2, i = rr & 3;
  const int lane = (d & 15) + 16 * a;
  return (((d >> 4) * 2 + s) * 64 + lane) * 8 + 4 * half + i;
}
__host__ __device__ __forceinline__ int vtile_frag(int dt, int s, int lane) {
  return ((dt * 2 + s) * 64 + lane) * 8;
}

// ---------------------------------------------------------------- wave helpers

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sums over the 16 lanes of each DPP row of eight values per lane, with the
// totals spread back over the row (reduce-scatter by halving, no branches):
// v[h][i] is the lane's term of item 4h + i. A lane whose position in its
// row is c receives the total of item 4·c₃ + 2·c₀ + c₁ (cₖ = bit k of c);
// lanes c and c ^ 4 receive the same item. 23 VALU operations against 32 for
// eight full row sums.
__device__ __forceinline__ float row_scatter_sum8(const f32x4 (&v)[2], int c) {
  const bool b3 = (c & 8) != 0, b0 = (c & 1) != 0, b1 = (c & 2) != 0;
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // partner c ^ 8 keeps the other half
    const float send = b3 ? v[0][i] : v[1][i];
    const float keep = b3 ? v[1][i] : v[0][i];
    a[i] = keep + dpp_f<0x128>(send);  // row_ror:8
  }
  float b[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // partner c ^ 1
    const float send = b0 ? a[k] : a[k + 2];
    const float keep = b0 ? a[k + 2] : a[k];
    b[k] = keep + dpp_f<0xB1>(send);  // quad_perm [1,0,3,2]
  }
  const float send = b1 ? b[0] : b[1];  // partner c ^ 2
  const float keep = b1 ? b[1] : b[0];
  const float d = keep + dpp_f<0x4E>(send);  // quad_perm [2,3,0,1]
  return d + dpp_f<0x1B>(dpp_f<0x141>(d));  // + lane c ^ 4: row_half_mirror, quad_perm [3,2,1,0]
}

// The value of lane l ^ 16 / l ^ 32, from the gfx950 lane swaps (no LDS):
// swapping a value with itself leaves r[0] holding the even rows (resp. the
// low half) twice and r[1] the odd rows (the high half) twice.
__device__ __forceinline__ float xor16_f(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32_f(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (same column, all keys).
__device__ __forceinline__ float col_max4(float v) {
  v = fmaxf(v, xor16_f(v));
  return fmaxf(v, xor32_f(v));
}
__device__ __forceinline__ float col_sum4(float v) {
  v += xor16_f(v);
  return v + xor32_f(v);
}

// A fragment read from p where ok, zeros elsewhere. p must be readable in
// every lane (callers clamp the indices), so the read is unconditional: the
// reads of a loop then stay in flight together instead of each sitting in a
// branch of its own that the compiler waits on.
template <class T>
__device__ __forceinline__ Frag<T> frag_load_if(const typename T::storage* p, bool ok) {
  const Frag<T> f = frag_load<T>(p);
  return ok ? f : frag_zero<T>();
}

// Direct global-to-LDS copy, 16 bytes per active lane: lane l's bytes land
// at lds + 16 l (lds must be the same in every lane). Tracked by vmcnt like a
// load; the compiler waits for it before the wave's next LDS read unless an
// explicit wait covers it first.
__device__ __forceinline__ void lds_copy16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// col_sum4 without the lane selects: a lane swap with the value as both
// operands returns the lane's own value in one half and its partner's in the
// other, so their sum is the pair's sum in every lane. Floating-point
// addition is commutative, so the result equals col_sum4's bit for bit.
__device__ __forceinline__ float col_sum4_fast(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Workgroup barrier that orders LDS accesses only: outstanding global loads
// and stores stay in flight across it (__syncthreads waits for all of them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS accesses before the following ones.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy softmax rescaling: the running maximum (log2 units) is only raised
// when a new logit exceeds it by more than this, so probabilities stay below
// 2^kLazyMax and most steps need neither a cross-lane max nor a rescale.
constexpr float kLazyMax = 8.0f;

// True when any lane of the wave holds v != 0 (wave-uniform).
__device__ __forceinline__ bool wave_any(bool v) { return __ballot(v) != 0; }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// One 32-key step of an online-softmax attention for one 16-column query
// tile: st holds the raw S^T of keys [kbase, kbase+32) in C layout; with MASK,
// keys outside [klo, khi] are excluded. Updates m and l, rescales acc when m
// moves, and returns the probabilities as the B operand of the P.V product.
// m is raised lazily (kLazyMax); the final output is acc / l whatever m is.
template <class T, int DT, bool MASK>
__device__ __forceinline__ Frag<T> online_probs(f32x4 (&st)[2], int kbase, int klo, int khi, int grp,
                                                float sl2, float& m, float& l, f32x4 (&acc)[DT]) {
  // The maximum is taken over the raw scores (sl2 > 0), and the scaling is
  // folded into the exponent: p = 2^(s sl2 - m).
  float lmx = -INFINITY;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = st[h2][i];
      if (MASK) {
        const int key = kbase + 16 * h2 + 4 * grp + i;
        x = (key >= klo && key <= khi) ? x : -INFINITY;
      }
      st[h2][i] = x;
      lmx = fmaxf(lmx, x);
    }
  lmx = fmaxf(lmx * sl2, kNegBig);
  if (wave_any(lmx > m + kLazyMax)) {
    const float mn = fmaxf(m, col_max4(lmx));
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    m = mn;
  }
  float sum = 0.f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(fmaf(st[h2][i], sl2, -m));
      st[h2][i] = p;
      sum += p;
    }
  l += sum;
  return pack_p<T>(st[0], st[1]);
}

// online_probs followed by acc += V^T . P^T with the V^T fragments vf.
template <class T, int DT, bool MASK>
__device__ __forceinline__ void online_step(f32x4 (&st)[2], int kbase, int klo, int khi, int grp,
                                            float sl2, float& m, float& l, f32x4 (&acc)[DT],
                                            const Frag<T> (&vf)[DT]) {
  const Frag<T> pf = online_probs<T, DT, MASK>(st, kbase, klo, khi, grp, sl2, m, l, acc);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) mma(acc[dt], vf[dt], pf);
}

}  // namespace nsa
