// Host side of libnsa: argument validation, workspace layout and the launch
// sequence of each entry point. Every check runs before anything is
// enqueued; a failing call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "nsa.h"
#include "nsa_internal.h"
#include "nsa_backward.h"

namespace {

thread_local std::string g_last_error;

nsa_status_t fail(nsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

nsa_status_t ok() {
  g_last_error.clear();
  return NSA_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(nsa_dtype_t d) { return d == NSA_F32 || d == NSA_BF16; }

// general: the prefill's block sizes (l <= l', l' a multiple of 32);
// otherwise (decode, backward) both must be 64.
nsa_status_t check_params(const nsa_params_t* p, int head_dim, bool general = false) {
  if (p == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->compress_block_size < 1 || p->select_block_size < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "block sizes must be >= 1 (got %d, %d)",
                p->compress_block_size, p->select_block_size);
  if (p->select_top_k < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "select_top_k must be >= 1 (got %d)", p->select_top_k);
  if (p->sliding_window < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "sliding_window must be >= 1 (got %d)", p->sliding_window);
  if (!std::isfinite(p->softmax_scale))
    return fail(NSA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  if (p->select_top_k > 64)
    return fail(NSA_ERR_UNSUPPORTED, "select_top_k > 64 is not supported (got %d)", p->select_top_k);
  const int l = p->compress_block_size, ls = p->select_block_size;
  if (!general) {
    if (l != nsa::kBlock || ls != nsa::kBlock)
      return fail(NSA_ERR_UNSUPPORTED, "this entry point needs compress_block_size == select_block_size == 64 "
                                       "(got %d, %d)", l, ls);
  } else {
    if (ls < l)
      return fail(NSA_ERR_UNSUPPORTED, "select_block_size (%d) below compress_block_size (%d) is not supported",
                  ls, l);
    if (ls % 32 != 0)
      return fail(NSA_ERR_UNSUPPORTED, "select_block_size must be a multiple of 32 (got %d)", ls);
    if (static_cast<int64_t>(ls) * p->select_top_k > nsa::kMaxSelTokens)
      return fail(NSA_ERR_UNSUPPORTED, "select_top_k * select_block_size above %d is not supported (got %d * %d)",
                  nsa::kMaxSelTokens, p->select_top_k, ls);
    if (l > 4096) return fail(NSA_ERR_UNSUPPORTED, "compress_block_size above 4096 is not supported (got %d)", l);
  }
  (void)head_dim;
  return NSA_OK;
}

// Geometry of a prefill call beyond nsa_params_t: the compression stride and
// the optional learned compressor / gate layer (all null: block means, gates
// given).
struct Geometry {
  int stride;  // d (the compress block size when not given)
  const nsa_general_t* gen;
  bool learned() const { return gen != nullptr && (gen->wk != nullptr || gen->wv != nullptr); }
  bool gate_layer() const { return gen != nullptr && gen->gate_w != nullptr; }
};

nsa_status_t check_general(const nsa_params_t* p, const nsa_general_t* gen, Geometry* geo) {
  geo->gen = gen;
  geo->stride = p->compress_block_size;
  if (gen == nullptr) return NSA_OK;
  if (gen->compress_stride < 1 || gen->compress_stride > p->compress_block_size)
    return fail(NSA_ERR_INVALID_ARGUMENT, "compress_stride must lie in [1, compress_block_size %d] (got %d)",
                p->compress_block_size, gen->compress_stride);
  geo->stride = gen->compress_stride;
  if ((gen->wk == nullptr) != (gen->bk == nullptr) || (gen->wv == nullptr) != (gen->bv == nullptr) ||
      (gen->wk == nullptr) != (gen->wv == nullptr))
    return fail(NSA_ERR_INVALID_ARGUMENT, "the learned compressor needs all of wk, bk, wv, bv (or none)");
  if ((gen->gate_w == nullptr) != (gen->gate_b == nullptr))
    return fail(NSA_ERR_INVALID_ARGUMENT, "the gate layer needs both gate_w and gate_b (or neither)");
  if ((gen->wk != nullptr && (!aligned16(gen->wk) || !aligned16(gen->wv))) ||
      (gen->gate_w != nullptr && (reinterpret_cast<uintptr_t>(gen->gate_w) & 1u)))
    return fail(NSA_ERR_INVALID_ARGUMENT, "wk / wv must be 16-byte aligned and gate_w element aligned");
  return NSA_OK;
}

nsa_status_t check_heads(int hq, int g, int d) {
  if (hq < 1 || g < 1 || d < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "n_q_heads, n_kv_heads, head_dim must be >= 1");
  if (hq % g != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", hq, g);
  if (hq / g > 16)
    return fail(NSA_ERR_UNSUPPORTED, "more than 16 query heads per KV head (%d) is not supported", hq / g);
  if (d != 64 && d != 128)
    return fail(NSA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d);
  return NSA_OK;
}

nsa_status_t check_dtypes(nsa_dtype_t in, nsa_dtype_t out) {
  if (!dtype_ok(in) || !dtype_ok(out)) return fail(NSA_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (in == NSA_F32 && out == NSA_BF16)
    return fail(NSA_ERR_UNSUPPORTED, "f32 input with bf16 output is not supported");
  return NSA_OK;
}

nsa_status_t check_strides(const char* name, const int64_t* s, int n, bool vec8) {
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(NSA_ERR_INVALID_ARGUMENT, "%s stride[%d] is negative", name, i);
    if (vec8 && (s[i] % 8) != 0)
      return fail(NSA_ERR_INVALID_ARGUMENT, "%s stride[%d] = %lld is not a multiple of 8 elements",
                  name, i, static_cast<long long>(s[i]));
  }
  return NSA_OK;
}

nsa_status_t check_ptr(const char* name, const void* p, bool need16) {
  if (p == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (need16 && !aligned16(p)) return fail(NSA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return NSA_OK;
}

#define NSA_TRY(expr)              \
  do {                             \
    nsa_status_t st_ = (expr);     \
    if (st_ != NSA_OK) return st_; \
  } while (0)

// ------------------------------------------------------------------ prefill

struct PrefillPlan {
  int Nb, Nc, NcT, cmp_waves, cmp_lo_lds, cmp_gsc, cmp_tiles, sel_tiles, sel_pf;
  size_t off_kt, off_vt, off_kct, off_kclt, off_vct, off_idx, off_part, off_gates, off_cmp_sc, total;
};

// q_offset: the queries are positions [q_offset, seqlen) (0 for a whole
// prefill); only the tile counts depend on it, not the workspace.
nsa_status_t plan_prefill(const nsa_prefill_desc_t* d, const nsa_params_t* p, PrefillPlan* pl,
                          int64_t q_offset = 0, const nsa_general_t* gen = nullptr, Geometry* geo_out = nullptr) {
  if (d == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0 || d->seqlen < 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "batch and seqlen must be >= 0");
  NSA_TRY(check_heads(d->n_q_heads, d->n_kv_heads, d->head_dim));
  NSA_TRY(check_dtypes(d->in_dtype, d->out_dtype));
  NSA_TRY(check_params(p, d->head_dim, true));
  Geometry geo;
  NSA_TRY(check_general(p, gen, &geo));
  if (geo_out != nullptr) *geo_out = geo;
  NSA_TRY(check_strides("q", d->q_stride, 3, true));
  NSA_TRY(check_strides("k", d->k_stride, 3, true));
  NSA_TRY(check_strides("v", d->v_stride, 3, true));
  NSA_TRY(check_strides("gates", d->g_stride, 3, false));
  NSA_TRY(check_strides("out", d->o_stride, 3, true));
  const int64_t B = d->batch, L = d->seqlen, G = d->n_kv_heads, D = d->head_dim;
  if (B * L * d->n_q_heads > INT32_MAX || B * L * G * p->select_top_k > INT32_MAX ||
      B * G * ((L + 63) / 64) * 64 > INT32_MAX)
    return fail(NSA_ERR_UNSUPPORTED, "problem too large for 32-bit work indexing");
  pl->Nb = static_cast<int>((L + 63) / 64);
  const int64_t cl = p->compress_block_size;
  pl->Nc = static_cast<int>(L >= cl ? (L - cl) / geo.stride + 1 : 0);
  pl->NcT = (pl->Nc + 63) / 64;
  if (B * G * static_cast<int64_t>(pl->NcT) * 64 > INT32_MAX)
    return fail(NSA_ERR_UNSUPPORTED, "problem too large for 32-bit work indexing");
  // the compressed kernel runs 8 waves per workgroup (its two-segment
  // schedule); the low parts of the K means go through LDS as well when that
  // still fits, and the tokens' block-score rows stay in LDS when they fit,
  // else in the workspace
  pl->cmp_waves = 8;
  pl->cmp_lo_lds = 0;
  pl->cmp_gsc = 1;
  const bool bf16 = d->in_dtype == NSA_BF16;
  for (int gsc = 0; gsc <= 1 && pl->cmp_gsc == 1; ++gsc)
    for (int lol = bf16 ? 1 : 0; lol >= 0; --lol)
      if (nsa::cmpwin_lds_bytes(8, gsc ? 0 : pl->NcT, static_cast<int>(D), bf16, lol != 0) <=
          static_cast<size_t>(nsa::kMaxLds)) {
        pl->cmp_lo_lds = lol;
        pl->cmp_gsc = gsc;
        break;
      }
  const size_t sel_stat = nsa::sel_static_lds_bytes(static_cast<int>(D), d->in_dtype == NSA_BF16);
  pl->sel_pf = nsa::sel_lds_bytes(pl->Nb, static_cast<int>(D), d->in_dtype == NSA_BF16, true) + sel_stat <=
                       static_cast<size_t>(nsa::kMaxLds)
                   ? 1
                   : 0;
  if (nsa::sel_lds_bytes(pl->Nb, static_cast<int>(D), d->in_dtype == NSA_BF16, false) + sel_stat >
      static_cast<size_t>(nsa::kMaxLds))
    return fail(NSA_ERR_UNSUPPORTED, "seqlen %lld needs more LDS for the selection lists than a CU has",
                static_cast<long long>(L));
  const int64_t tok_cmp = static_cast<int64_t>(pl->cmp_waves) * nsa::kCmpTPW;
  const int64_t tok_sel = 4 * static_cast<int64_t>(nsa::kSelTPW);
  const int64_t Lq = L - q_offset;
  pl->cmp_tiles = static_cast<int>((Lq + tok_cmp - 1) / tok_cmp);
  pl->sel_tiles = static_cast<int>((Lq + tok_sel - 1) / tok_sel);
  const size_t elem = d->in_dtype == NSA_BF16 ? 2 : 4;
  const size_t tile = 64 * static_cast<size_t>(D) * elem;
  size_t off = 0;
  pl->off_kt = off;
  off = align_up(off + static_cast<size_t>(B * G) * pl->Nb * tile);
  pl->off_vt = off;
  off = align_up(off + static_cast<size_t>(B * G) * pl->Nb * tile);
  pl->off_kct = off;
  off = align_up(off + static_cast<size_t>(B * G) * pl->NcT * tile);
  pl->off_kclt = off;  // low parts of the bf16 block means of K
  if (d->in_dtype == NSA_BF16) off = align_up(off + static_cast<size_t>(B * G) * pl->NcT * tile);
  pl->off_vct = off;
  off = align_up(off + static_cast<size_t>(B * G) * pl->NcT * tile);
  pl->off_idx = off;
  off = align_up(off + static_cast<size_t>(B * L * G) * p->select_top_k * sizeof(int32_t));
  // bf16 output: fp32 rows of the window + compressed part, so that the
  // output is rounded once (the query rows never exceed the context length)
  pl->off_part = off;
  if (d->out_dtype == NSA_BF16) off = align_up(off + static_cast<size_t>(B * L * d->n_q_heads) * D * sizeof(float));
  // gate layer: its fp32 gates of every query row
  pl->off_gates = off;
  if (geo.gate_layer()) off = align_up(off + static_cast<size_t>(B * L * d->n_q_heads) * 3 * sizeof(float));
  // block-score rows of the compressed kernel when they do not fit LDS
  pl->off_cmp_sc = off;
  if (pl->cmp_gsc) off = align_up(off + static_cast<size_t>(B * G) * (L + 2) * pl->NcT * 64 * sizeof(float));
  pl->total = off;
  return NSA_OK;
}

// ------------------------------------------------------------------ backward

struct BwdPlan {
  int Nb, Nc, NcT, units[3];
  size_t off_ka, off_kv, off_va, off_vv, off_kcm, off_vcm, off_kca, off_kcv, off_vca, off_vcv;
  size_t off_qT, off_dT, off_dN, off_stat, off_dkc, off_dvc, off_cnt, off_offs, off_pofs, off_list, total;
};

nsa_status_t plan_backward(const nsa_prefill_desc_t* d, const nsa_params_t* p, BwdPlan* pl) {
  if (d == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0 || d->seqlen < 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "batch and seqlen must be >= 0");
  NSA_TRY(check_heads(d->n_q_heads, d->n_kv_heads, d->head_dim));
  NSA_TRY(check_dtypes(d->in_dtype, d->out_dtype));
  NSA_TRY(check_params(p, d->head_dim));
  NSA_TRY(check_strides("q", d->q_stride, 3, true));
  NSA_TRY(check_strides("k", d->k_stride, 3, true));
  NSA_TRY(check_strides("v", d->v_stride, 3, true));
  NSA_TRY(check_strides("gates", d->g_stride, 3, false));
  NSA_TRY(check_strides("dout", d->o_stride, 3, false));
  const int64_t B = d->batch, L = d->seqlen, G = d->n_kv_heads, D = d->head_dim, Hq = d->n_q_heads;
  if (B * L * Hq * D > INT32_MAX * 4LL || B * L * G * p->select_top_k > INT32_MAX ||
      B * G * ((L + 63) / 64) * 64 > INT32_MAX || B * L * G > INT32_MAX / 16)
    return fail(NSA_ERR_UNSUPPORTED, "problem too large for 32-bit work indexing");
  pl->Nb = static_cast<int>((L + 63) / 64);
  pl->Nc = static_cast<int>(L / 64);
  pl->NcT = (pl->Nc + 63) / 64;
  // key-side workgroups per (sequence, group): compressed, pieces of
  // kBwdCmpPiece tokens of [64*64c + 63, L) per 64-mean chunk; selected, at
  // most one piece per block plus one per kBwdSelPiece list entries; window,
  // one per 64-key chunk (its 63 + w tokens)
  const int64_t cmp_pieces = std::max<int64_t>(1, (L + nsa::kBwdCmpPiece - 1) / nsa::kBwdCmpPiece);
  pl->units[0] = static_cast<int>(pl->NcT * cmp_pieces);
  pl->units[1] = static_cast<int>(pl->Nb + (L * p->select_top_k + nsa::kBwdSelPiece - 1) / nsa::kBwdSelPiece);
  pl->units[2] = pl->Nb;
  if (B * G * std::max<int64_t>(pl->units[0], pl->units[1]) > INT32_MAX)
    return fail(NSA_ERR_UNSUPPORTED, "problem too large for 32-bit work indexing");
  const size_t elem = d->in_dtype == NSA_BF16 ? 2 : 4;
  const size_t tiles = static_cast<size_t>(B * G) * pl->Nb * 64 * D * elem;
  const size_t ctiles = static_cast<size_t>(B * G) * pl->NcT * 64 * D * elem;
  const size_t means = static_cast<size_t>(B) * pl->Nc * G * D * elem;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  pl->off_ka = take(tiles);
  pl->off_kv = take(tiles);
  pl->off_va = take(tiles);
  pl->off_vv = take(tiles);
  pl->off_kcm = take(means);
  pl->off_vcm = take(means);
  pl->off_kca = take(ctiles);
  pl->off_kcv = take(ctiles);
  pl->off_vca = take(ctiles);
  pl->off_vcv = take(ctiles);
  pl->off_qT = take(static_cast<size_t>(B * L * G) * D * 16 * elem);
  pl->off_dT = take(static_cast<size_t>(B * L * G) * D * 16 * elem);
  pl->off_dN = take(static_cast<size_t>(B * L * Hq) * D * elem);
  pl->off_stat = take(static_cast<size_t>(B * L * Hq) * 3 * 2 * sizeof(float));
  pl->off_dkc = take(static_cast<size_t>(B) * pl->Nc * G * D * sizeof(float));
  pl->off_dvc = take(static_cast<size_t>(B) * pl->Nc * G * D * sizeof(float));
  pl->off_cnt = take(static_cast<size_t>(B * G) * pl->Nb * sizeof(int32_t));
  pl->off_offs = take(static_cast<size_t>(B * G) * (pl->Nb + 1) * sizeof(int32_t));
  pl->off_pofs = take(static_cast<size_t>(B * G) * (pl->Nb + 1) * sizeof(int32_t));
  pl->off_list = take(static_cast<size_t>(B * G * L) * p->select_top_k * sizeof(int32_t));
  pl->total = off;
  return NSA_OK;
}

// ------------------------------------------------------------------ decode

struct DecodePlan {
  int NmaxPad;
  bool logits_lds;
  size_t off_logits, off_idx, off_gates, total;
};

// general: the general-geometry entry points (gen may then be NULL: the
// plain stride, gates given); geo_out receives the geometry.
nsa_status_t plan_decode(const nsa_decode_desc_t* d, const nsa_params_t* p, DecodePlan* pl, bool general = false,
                         const nsa_general_t* gen = nullptr, Geometry* geo_out = nullptr) {
  if (d == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0) return fail(NSA_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  if (d->max_seqlen < 1) return fail(NSA_ERR_INVALID_ARGUMENT, "max_seqlen must be >= 1");
  if (d->max_blocks < 0) return fail(NSA_ERR_INVALID_ARGUMENT, "max_blocks must be >= 0");
  NSA_TRY(check_heads(d->n_q_heads, d->n_kv_heads, d->head_dim));
  NSA_TRY(check_dtypes(d->in_dtype, d->out_dtype));
  NSA_TRY(check_params(p, d->head_dim, general));
  Geometry geo;
  NSA_TRY(check_general(p, general ? gen : nullptr, &geo));
  if (geo_out != nullptr) *geo_out = geo;
  // compressed blocks of the longest sequence (the cache rows a call may read)
  const int cl = p->compress_block_size;
  const int nv = d->max_seqlen >= cl ? (d->max_seqlen - cl) / geo.stride + 1 : 0;
  if (d->max_blocks < nv)
    return fail(NSA_ERR_INVALID_ARGUMENT, "max_blocks (%d) < the %d compressed blocks of max_seqlen %d",
                d->max_blocks, nv, d->max_seqlen);
  NSA_TRY(check_strides("q", d->q_stride, 2, true));
  NSA_TRY(check_strides("k_cache", d->k_stride, 3, true));
  NSA_TRY(check_strides("v_cache", d->v_stride, 3, true));
  NSA_TRY(check_strides("kc_cache", d->kc_stride, 3, true));
  NSA_TRY(check_strides("vc_cache", d->vc_stride, 3, true));
  NSA_TRY(check_strides("gates", d->g_stride, 2, false));
  NSA_TRY(check_strides("out", d->o_stride, 2, false));
  const int64_t B = d->batch, G = d->n_kv_heads, D = d->head_dim;
  pl->NmaxPad = (nv + 63) / 64 * 64;
  if (B * G > INT32_MAX / 16)
    return fail(NSA_ERR_UNSUPPORTED, "batch * n_kv_heads too large");
  const bool bf16 = d->in_dtype == NSA_BF16;
  if (nsa::dec_lds_bytes(pl->NmaxPad, static_cast<int>(D), bf16, false) > static_cast<size_t>(nsa::kMaxLds))
    return fail(NSA_ERR_UNSUPPORTED, "max_seqlen %d needs more LDS for block scores than a CU has",
                d->max_seqlen);
  pl->logits_lds =
      nsa::dec_lds_bytes(pl->NmaxPad, static_cast<int>(D), bf16, true) <= static_cast<size_t>(nsa::kMaxLds);
  size_t off = 0;
  pl->off_logits = off;
  if (!pl->logits_lds) off = align_up(off + static_cast<size_t>(B * G) * 16 * pl->NmaxPad * sizeof(float));
  pl->off_idx = off;
  off = align_up(off + static_cast<size_t>(B * G) * p->select_top_k * sizeof(int32_t));
  // gate layer: its fp32 gates of every sequence and head
  pl->off_gates = off;
  if (geo.gate_layer()) off = align_up(off + static_cast<size_t>(B * d->n_q_heads) * 3 * sizeof(float));
  pl->total = off;
  return NSA_OK;
}

float scale_log2(const nsa_params_t* p, int D) {
  const float s = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt(static_cast<float>(D));
  return s * nsa::kLog2eHost;
}

}  // namespace

extern "C" {

const char* nsa_status_string(nsa_status_t status) {
  switch (status) {
    case NSA_OK:
      return "NSA_OK";
    case NSA_ERR_INVALID_ARGUMENT:
      return "NSA_ERR_INVALID_ARGUMENT";
    case NSA_ERR_UNSUPPORTED:
      return "NSA_ERR_UNSUPPORTED";
    case NSA_ERR_WORKSPACE_TOO_SMALL:
      return "NSA_ERR_WORKSPACE_TOO_SMALL";
    case NSA_ERR_HIP:
      return "NSA_ERR_HIP";
  }
  return "NSA_ERR_UNKNOWN";
}

const char* nsa_last_error(void) { return g_last_error.c_str(); }

int32_t nsa_version(void) { return 100; }

nsa_status_t nsa_prefill_workspace_bytes(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                         size_t* bytes) {
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  PrefillPlan pl;
  NSA_TRY(plan_prefill(desc, params, &pl));
  *bytes = pl.total;
  return ok();
}

nsa_status_t nsa_decode_workspace_bytes(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                        size_t* bytes) {
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DecodePlan pl;
  NSA_TRY(plan_decode(desc, params, &pl));
  *bytes = pl.total;
  return ok();
}

// Splits of a KV group's (sequence, tile) items of the selected-block kernel
// over the group's 8 / G XCDs, for a whole prefill: equal contiguous shares,
// except for one sequence longer than 32768 tokens shared by two XCDs, where
// the first XCD (the earlier tokens, whose blocks come from a shorter
// context) takes 57 % of the tiles. Measured at 64k (k_sel, ms, one box):
// 50 % 7.72, 55 % 7.48-7.69, 56 % 7.82-7.86, 57 % 7.29-7.30, 57.5 % 7.50-7.55,
// 58 % 7.90, 60 % 7.79; 57 % was 5-7 % faster than 50 % on every box
// tried. The dependence is not smooth, so no model is fitted; at 32k the
// best split measured (55 %) gained ~3 % and is not used.
static void sel_split(int B, int G, int T, int L, bool interleave, int* bounds) {
  bounds[0] = -1;
  if (interleave || G <= 0 || 8 % G != 0 || T <= 0) return;
  const int pg = 8 / G;
  const int64_t n_items = static_cast<int64_t>(B) * T;
  for (int k = 0; k <= pg; ++k) bounds[k] = static_cast<int>(n_items * k / pg);
  if (pg == 2 && B == 1 && L > 32768) bounds[1] = static_cast<int>((static_cast<int64_t>(T) * 57 + 99) / 100);
}

// Sequences: either one query range [q_offset, seqlen) for every sequence
// (seq_lens == nullptr), or per-sequence device arrays seq_lens / q_offsets
// with q_offset = seqlen - (rows of the query arrays).
static nsa_status_t prefill_impl(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                 int64_t q_offset, const int32_t* seq_lens, const int32_t* q_offsets,
                                 const void* q, const void* k, const void* v, const void* gates,
                                 void* out, int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* events,
                                 void* save_o = nullptr, float* save_lse = nullptr,
                                 const nsa_general_t* gen = nullptr) {
  if (desc == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (q_offset < 0 || q_offset > desc->seqlen)
    return fail(NSA_ERR_INVALID_ARGUMENT, "q_offset %lld outside [0, seqlen %d]",
                static_cast<long long>(q_offset), desc->seqlen);
  PrefillPlan pl;
  Geometry geo;
  NSA_TRY(plan_prefill(desc, params, &pl, q_offset, gen, &geo));
  if (save_o != nullptr &&
      (params->compress_block_size != nsa::kBlock || params->select_block_size != nsa::kBlock ||
       geo.stride != nsa::kBlock || geo.learned() || geo.gate_layer()))
    return fail(NSA_ERR_UNSUPPORTED, "keeping the selected branch for the backward needs the plain geometry "
                                     "(blocks of 64, stride 64, block means, given gates)");
  if (idx_mode != NSA_IDX_COMPUTE && idx_mode != NSA_IDX_INJECT)
    return fail(NSA_ERR_INVALID_ARGUMENT, "unknown idx_mode %d", static_cast<int>(idx_mode));
  // empty input or no query rows: nothing to do
  if (desc->batch == 0 || desc->seqlen == 0 || q_offset == desc->seqlen) return ok();
  if (seq_lens != nullptr) {
    NSA_TRY(check_ptr("seq_lens", seq_lens, false));
    if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(q_offsets) & 3u) != 0)
      return fail(NSA_ERR_INVALID_ARGUMENT, "seq_lens / q_offsets are not 4-byte aligned");
  }
  NSA_TRY(check_ptr("q", q, true));
  NSA_TRY(check_ptr("k", k, true));
  NSA_TRY(check_ptr("v", v, true));
  if (!geo.gate_layer()) NSA_TRY(check_ptr("gates", gates, false));
  NSA_TRY(check_ptr("out", out, true));
  NSA_TRY(check_ptr("workspace", workspace, true));
  if (idx_mode == NSA_IDX_INJECT && idx == nullptr)
    return fail(NSA_ERR_INVALID_ARGUMENT, "NSA_IDX_INJECT needs idx");
  if (idx != nullptr && (reinterpret_cast<uintptr_t>(idx) & 3u) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "idx is not 4-byte aligned");
  const size_t gal = desc->in_dtype == NSA_BF16 ? 2 : 4;
  if (!geo.gate_layer() && (reinterpret_cast<uintptr_t>(gates) % gal) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "gates is not aligned to its element size");
  if (workspace_bytes < pl.total)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.total,
                workspace_bytes);

  nsa::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = desc->batch;
  a.L = desc->seqlen;
  a.t0 = seq_lens != nullptr ? 0 : static_cast<int>(q_offset);
  a.Lq = desc->seqlen - static_cast<int>(q_offset);
  a.seq_lens = seq_lens;
  a.q_offs = seq_lens != nullptr ? q_offsets : nullptr;
  // k_sel's XCD mapping: contiguous for a whole prefill, interleaved for
  // chunks and varlen batches (and only where the groups divide the XCDs)
  a.sel_interleave = (seq_lens != nullptr || q_offset > 0) && 8 % desc->n_kv_heads == 0 ? 1 : 0;
  sel_split(desc->batch, desc->n_kv_heads, pl.sel_tiles, desc->seqlen, a.sel_interleave != 0, a.sel_bounds);
  a.Hq = desc->n_q_heads;
  a.G = desc->n_kv_heads;
  a.Hg = a.Hq / a.G;
  a.D = desc->head_dim;
  a.n = params->select_top_k;
  a.w = params->sliding_window;
  a.Nb = pl.Nb;
  a.Nc = pl.Nc;
  a.NcT = pl.NcT;
  a.cmp_waves = pl.cmp_waves;
  a.cmp_lo_lds = pl.cmp_lo_lds;
  a.cmp_tiles = pl.cmp_tiles;
  a.sel_tiles = pl.sel_tiles;
  a.sel_bm_words = nsa::sel_bm_words(pl.Nb);
  a.sel_pf = pl.sel_pf;
  a.scale_log2 = scale_log2(params, a.D);
  a.inject = idx_mode == NSA_IDX_INJECT ? 1 : 0;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gates = gates;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.idx = idx != nullptr ? idx : reinterpret_cast<int32_t*>(ws + pl.off_idx);
  a.kt = ws + pl.off_kt;
  a.vt = ws + pl.off_vt;
  a.save_o = save_o;
  a.save_lse = save_lse;
  a.part = desc->out_dtype == NSA_BF16 ? reinterpret_cast<float*>(ws + pl.off_part) : nullptr;
  a.cl = params->compress_block_size;
  a.cd = geo.stride;
  a.ls = params->select_block_size;
  a.inv_cl = 1.0f / static_cast<float>(a.cl);
  a.sel_map = !(a.cl == a.cd && a.cd == a.ls) ? 1 : 0;
  a.cmp_in_prep = (a.cl == nsa::kBlock && a.cd == nsa::kBlock && !geo.learned()) ? 1 : 0;
  if (geo.learned()) {
    a.wk = gen->wk;
    a.bk = gen->bk;
    a.wv = gen->wv;
    a.bv = gen->bv;
  }
  if (geo.gate_layer()) {
    a.gate_w = gen->gate_w;
    a.gate_b = gen->gate_b;
    a.gates32 = reinterpret_cast<float*>(ws + pl.off_gates);
  }
  a.kct = ws + pl.off_kct;
  a.kclt = ws + pl.off_kclt;
  a.vct = ws + pl.off_vct;
  a.cmp_sc = pl.cmp_gsc ? reinterpret_cast<float*>(ws + pl.off_cmp_sc) : nullptr;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = desc->q_stride[i];
    a.ks[i] = desc->k_stride[i];
    a.vs[i] = desc->v_stride[i];
    a.gs[i] = desc->g_stride[i];
    a.os[i] = desc->o_stride[i];
  }
  hipError_t e = nsa::launch_prefill(a, desc->in_dtype == NSA_BF16, desc->out_dtype == NSA_BF16,
                                     static_cast<hipStream_t>(stream),
                                     reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "HIP error in prefill launch: %s", hipGetErrorString(e));
  return ok();
}

nsa_status_t nsa_fwd_prefill(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                             const void* q, const void* k, const void* v, const void* gates,
                             void* out, int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return prefill_impl(desc, params, 0, nullptr, nullptr, q, k, v, gates, out, idx, idx_mode, workspace,
                      workspace_bytes, stream, nullptr);
}

nsa_status_t nsa_prefill_general_workspace_bytes(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                                 const nsa_general_t* general, size_t* bytes) {
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  PrefillPlan pl;
  NSA_TRY(plan_prefill(desc, params, &pl, 0, general));
  *bytes = pl.total;
  return ok();
}

nsa_status_t nsa_fwd_prefill_general(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                     const nsa_general_t* general, const void* q, const void* k, const void* v,
                                     const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(desc, params, 0, nullptr, nullptr, q, k, v, gates, out, idx, idx_mode, workspace,
                      workspace_bytes, stream, nullptr, nullptr, nullptr, general);
}

nsa_status_t nsa_fwd_prefill_save(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                  const void* k, const void* v, const void* gates, void* out, int32_t* idx,
                                  nsa_idx_mode_t idx_mode, void* o_slc, float* lse_slc, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (desc != nullptr && desc->batch > 0 && desc->seqlen > 0) {
    NSA_TRY(check_ptr("o_slc", o_slc, true));
    NSA_TRY(check_ptr("lse_slc", lse_slc, false));
    if ((reinterpret_cast<uintptr_t>(lse_slc) & 3u) != 0)
      return fail(NSA_ERR_INVALID_ARGUMENT, "lse_slc is not 4-byte aligned");
  }
  return prefill_impl(desc, params, 0, nullptr, nullptr, q, k, v, gates, out, idx, idx_mode, workspace,
                      workspace_bytes, stream, nullptr, o_slc, lse_slc);
}

nsa_status_t nsa_fwd_prefill_chunk(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                   int32_t q_offset, const void* q, const void* k, const void* v,
                                   const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(desc, params, q_offset, nullptr, nullptr, q, k, v, gates, out, idx, idx_mode,
                      workspace, workspace_bytes, stream, nullptr);
}

nsa_status_t nsa_fwd_prefill_varlen(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                    const int32_t* seq_lens, const int32_t* q_offsets,
                                    int32_t query_rows, const void* q, const void* k, const void* v,
                                    const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (desc == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (seq_lens == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "seq_lens is NULL");
  if (query_rows < 0 || query_rows > desc->seqlen)
    return fail(NSA_ERR_INVALID_ARGUMENT, "query_rows %d outside [0, seqlen %d]", query_rows, desc->seqlen);
  return prefill_impl(desc, params, static_cast<int64_t>(desc->seqlen) - query_rows, seq_lens, q_offsets, q, k,
                      v, gates, out, idx, idx_mode, workspace, workspace_bytes, stream, nullptr);
}

static nsa_status_t backward_impl(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                  const void* k, const void* v, const void* gates, const void* dout,
                                  const int32_t* idx, float* dq, float* dk, float* dv, float* dgates,
                                  void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                                  const void* o_slc = nullptr, const float* lse_slc = nullptr) {
  BwdPlan pl;
  NSA_TRY(plan_backward(desc, params, &pl));
  if (desc->batch == 0 || desc->seqlen == 0) return ok();
  NSA_TRY(check_ptr("q", q, true));
  NSA_TRY(check_ptr("k", k, true));
  NSA_TRY(check_ptr("v", v, true));
  NSA_TRY(check_ptr("gates", gates, false));
  NSA_TRY(check_ptr("dout", dout, false));
  NSA_TRY(check_ptr("idx", idx, false));
  NSA_TRY(check_ptr("dq", dq, true));
  NSA_TRY(check_ptr("dk", dk, false));
  NSA_TRY(check_ptr("dv", dv, false));
  NSA_TRY(check_ptr("dgates", dgates, false));
  NSA_TRY(check_ptr("workspace", workspace, true));
  const size_t gal = desc->in_dtype == NSA_BF16 ? 2 : 4, oal = desc->out_dtype == NSA_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(gates) % gal) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "gates is not aligned to its element size");
  if ((reinterpret_cast<uintptr_t>(dout) % oal) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "dout is not aligned to its element size");
  if ((reinterpret_cast<uintptr_t>(idx) & 3u) != 0 || (reinterpret_cast<uintptr_t>(dk) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(dv) & 3u) != 0 || (reinterpret_cast<uintptr_t>(dgates) & 3u) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "idx / dk / dv / dgates are not 4-byte aligned");
  if (workspace_bytes < pl.total)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.total, workspace_bytes);
  nsa::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = desc->batch;
  a.L = desc->seqlen;
  a.Hq = desc->n_q_heads;
  a.G = desc->n_kv_heads;
  a.Hg = a.Hq / a.G;
  a.D = desc->head_dim;
  a.n = params->select_top_k;
  a.w = params->sliding_window;
  a.Nb = pl.Nb;
  a.Nc = pl.Nc;
  a.NcT = pl.NcT;
  for (int i = 0; i < 3; ++i) a.bkv_units[i] = pl.units[i];
  a.scale_log2 = scale_log2(params, a.D);
  a.scale = a.scale_log2 / nsa::kLog2eHost;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gates = gates;
  a.dout = dout;
  a.idx = idx;
  a.o_slc = o_slc;
  a.lse_slc = lse_slc;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dgates = dgates;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = desc->q_stride[i];
    a.ks[i] = desc->k_stride[i];
    a.vs[i] = desc->v_stride[i];
    a.gs[i] = desc->g_stride[i];
    a.os[i] = desc->o_stride[i];
  }
  char* ws = static_cast<char*>(workspace);
  a.ka = ws + pl.off_ka;
  a.kv = ws + pl.off_kv;
  a.va = ws + pl.off_va;
  a.vv = ws + pl.off_vv;
  a.kcm = ws + pl.off_kcm;
  a.vcm = ws + pl.off_vcm;
  a.kca = ws + pl.off_kca;
  a.kcv = ws + pl.off_kcv;
  a.vca = ws + pl.off_vca;
  a.vcv = ws + pl.off_vcv;
  a.qT = ws + pl.off_qT;
  a.dT = ws + pl.off_dT;
  a.dN = ws + pl.off_dN;
  a.stat = reinterpret_cast<float2*>(ws + pl.off_stat);
  a.dkc = reinterpret_cast<float*>(ws + pl.off_dkc);
  a.dvc = reinterpret_cast<float*>(ws + pl.off_dvc);
  a.cnt = reinterpret_cast<int32_t*>(ws + pl.off_cnt);
  a.offs = reinterpret_cast<int32_t*>(ws + pl.off_offs);
  a.pofs = reinterpret_cast<int32_t*>(ws + pl.off_pofs);
  a.list = reinterpret_cast<int32_t*>(ws + pl.off_list);
  hipError_t e = nsa::launch_backward(a, desc->in_dtype == NSA_BF16, desc->out_dtype == NSA_BF16,
                                      static_cast<hipStream_t>(stream),
                                      reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "HIP error in backward launch: %s", hipGetErrorString(e));
  return ok();
}

nsa_status_t nsa_bwd_prefill_workspace_bytes(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                             size_t* bytes) {
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BwdPlan pl;
  NSA_TRY(plan_backward(desc, params, &pl));
  *bytes = pl.total;
  return ok();
}

nsa_status_t nsa_bwd_prefill(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                             const void* k, const void* v, const void* gates, const void* dout,
                             const int32_t* idx, float* dq, float* dk, float* dv, float* dgates,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(desc, params, q, k, v, gates, dout, idx, dq, dk, dv, dgates, workspace, workspace_bytes,
                       stream, nullptr);
}

nsa_status_t nsa_bwd_prefill_saved(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                   const void* k, const void* v, const void* gates, const void* dout,
                                   const int32_t* idx, const void* o_slc, const float* lse_slc, float* dq,
                                   float* dk, float* dv, float* dgates, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (desc != nullptr && desc->batch > 0 && desc->seqlen > 0) {
    NSA_TRY(check_ptr("o_slc", o_slc, true));
    NSA_TRY(check_ptr("lse_slc", lse_slc, false));
    if ((reinterpret_cast<uintptr_t>(lse_slc) & 3u) != 0)
      return fail(NSA_ERR_INVALID_ARGUMENT, "lse_slc is not 4-byte aligned");
  }
  return backward_impl(desc, params, q, k, v, gates, dout, idx, dq, dk, dv, dgates, workspace, workspace_bytes,
                       stream, nullptr, o_slc, lse_slc);
}

nsa_status_t nsa_bwd_prefill_saved_timed(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                         const void* q, const void* k, const void* v, const void* gates,
                                         const void* dout, const int32_t* idx, const void* o_slc,
                                         const float* lse_slc, float* dq, float* dk, float* dv, float* dgates,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         void* const* stage_events) {
  if (stage_events == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events is NULL");
  for (int i = 0; i <= nsa::kBwdStages; ++i)
    if (stage_events[i] == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events[%d] is NULL", i);
  if (desc != nullptr && desc->batch > 0 && desc->seqlen > 0) {
    NSA_TRY(check_ptr("o_slc", o_slc, true));
    NSA_TRY(check_ptr("lse_slc", lse_slc, false));
    if ((reinterpret_cast<uintptr_t>(lse_slc) & 3u) != 0)
      return fail(NSA_ERR_INVALID_ARGUMENT, "lse_slc is not 4-byte aligned");
  }
  return backward_impl(desc, params, q, k, v, gates, dout, idx, dq, dk, dv, dgates, workspace, workspace_bytes,
                       stream, stage_events, o_slc, lse_slc);
}

nsa_status_t nsa_bwd_prefill_timed(const nsa_prefill_desc_t* desc, const nsa_params_t* params, const void* q,
                                   const void* k, const void* v, const void* gates, const void* dout,
                                   const int32_t* idx, float* dq, float* dk, float* dv, float* dgates,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* stage_events) {
  if (stage_events == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events is NULL");
  for (int i = 0; i <= nsa::kBwdStages; ++i)
    if (stage_events[i] == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events[%d] is NULL", i);
  return backward_impl(desc, params, q, k, v, gates, dout, idx, dq, dk, dv, dgates, workspace, workspace_bytes,
                       stream, stage_events);
}

}  // extern "C"

// ------------------------------------------------------------------ token-level sparse attention (DSA)

namespace {

struct DsaPlan {
  int waves, heads_per_wave, topk_cache, parts, gpw, wg_waves;
  size_t off_scores, off_idx, total;
};

nsa_status_t plan_dsa(const nsa_dsa_desc_t* d, const nsa_dsa_params_t* p, DsaPlan* pl) {
  if (d == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (p == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (d->batch < 0 || d->seqlen < 0) return fail(NSA_ERR_INVALID_ARGUMENT, "batch and seqlen must be >= 0");
  const int Hq = d->n_q_heads, G = d->n_kv_heads, D = d->head_dim;
  if (Hq < 1 || G < 1 || D < 1 || d->idx_heads < 1 || d->idx_dim < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "head counts and dimensions must be >= 1");
  if (Hq % G != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", Hq, G);
  NSA_TRY(check_dtypes(d->in_dtype, d->out_dtype));
  if (p->top_k < 1) return fail(NSA_ERR_INVALID_ARGUMENT, "top_k must be >= 1 (got %d)", p->top_k);
  if (!std::isfinite(p->softmax_scale)) return fail(NSA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  if (D != 64 && D != 128) return fail(NSA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", D);
  if (d->idx_dim != 64 && d->idx_dim != 128)
    return fail(NSA_ERR_UNSUPPORTED, "idx_dim %d is not supported (64 or 128)", d->idx_dim);
  if (d->idx_heads > 16) return fail(NSA_ERR_UNSUPPORTED, "more than 16 indexer heads (%d)", d->idx_heads);
  if (p->top_k > nsa::kDsaMaxTopK)
    return fail(NSA_ERR_UNSUPPORTED, "top_k above %d is not supported (got %d)", nsa::kDsaMaxTopK, p->top_k);
  const int Hg = Hq / G;
  if (Hq > 64 || (Hg > 16 && Hg % 16 != 0))
    return fail(NSA_ERR_UNSUPPORTED, "needs n_q_heads <= 64 with at most 16 or a multiple of 16 query heads per "
                                     "KV head (got %d, %d)", Hq, Hg);
  NSA_TRY(check_strides("q", d->q_stride, 3, true));
  NSA_TRY(check_strides("k", d->k_stride, 3, true));
  NSA_TRY(check_strides("v", d->v_stride, 3, true));
  NSA_TRY(check_strides("out", d->o_stride, 3, true));
  NSA_TRY(check_strides("qi", d->qi_stride, 3, true));
  NSA_TRY(check_strides("ki", d->ki_stride, 2, true));
  NSA_TRY(check_strides("w", d->w_stride, 2, false));
  pl->waves = Hg >= 16 ? Hq / 16 : G;
  pl->heads_per_wave = Hg >= 16 ? 16 : Hg;
  const bool bf16 = d->in_dtype == NSA_BF16;
  // a query token's KV heads over as few attention workgroups as the LDS
  // allows: the most KV heads (a divisor of G) whose staging fits
  const int wpg = Hg >= 16 ? Hg / 16 : 1;
  const size_t lds_cap = static_cast<size_t>(nsa::kMaxLds) - 1024;   // room for the static LDS
  pl->gpw = 0;
  for (int gpw = G; gpw >= 1; --gpw)
    if (G % gpw == 0 && nsa::dsa_attn_lds_bytes(gpw, D, bf16, p->top_k) <= lds_cap) {
      pl->gpw = gpw;
      break;
    }
  if (pl->gpw == 0) return fail(NSA_ERR_UNSUPPORTED, "the attention stage of one KV head does not fit a CU's LDS");
  pl->parts = G / pl->gpw;
  pl->wg_waves = pl->gpw * wpg;
  pl->topk_cache = 65536;   // top 16 bits of a row's keys in LDS (128 KiB)
  if (d->seqlen > 131072)
    return fail(NSA_ERR_UNSUPPORTED, "seqlen above 131072 (the 128K context of the DSA how-to) is not supported "
                                     "(got %d)", d->seqlen);
  const int64_t B = d->batch, L = d->seqlen;
  if (B * L > INT32_MAX) return fail(NSA_ERR_UNSUPPORTED, "batch * seqlen too large");
  size_t off = 0;
  pl->off_scores = off;
  // the scores, then 64 floats where the indexer's lanes without a score to
  // write store (so its stores need no branch)
  off = align_up(off + static_cast<size_t>(B) * static_cast<size_t>(L) * static_cast<size_t>(L + 1) / 2 *
                           sizeof(float) +
                 64 * sizeof(float));
  pl->off_idx = off;
  off = align_up(off + static_cast<size_t>(B * L) * p->top_k * sizeof(int32_t));
  pl->total = off;
  return NSA_OK;
}

nsa_status_t dsa_impl(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, const void* q, const void* k,
                      const void* v, const void* qi, const void* ki, const void* w, void* out, int32_t* idx,
                      nsa_idx_mode_t idx_mode, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* events) {
  DsaPlan pl;
  NSA_TRY(plan_dsa(desc, params, &pl));
  if (idx_mode != NSA_IDX_COMPUTE && idx_mode != NSA_IDX_INJECT)
    return fail(NSA_ERR_INVALID_ARGUMENT, "unknown idx_mode %d", static_cast<int>(idx_mode));
  if (desc->batch == 0 || desc->seqlen == 0) return ok();
  const bool inject = idx_mode == NSA_IDX_INJECT;
  NSA_TRY(check_ptr("q", q, true));
  NSA_TRY(check_ptr("k", k, true));
  NSA_TRY(check_ptr("v", v, true));
  NSA_TRY(check_ptr("out", out, true));
  if (!inject) {
    NSA_TRY(check_ptr("qi", qi, true));
    NSA_TRY(check_ptr("ki", ki, true));
    NSA_TRY(check_ptr("w", w, false));
    const size_t el = desc->in_dtype == NSA_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(w) % el) != 0)
      return fail(NSA_ERR_INVALID_ARGUMENT, "w is not aligned to its element size");
  }
  NSA_TRY(check_ptr("workspace", workspace, true));
  if (inject && idx == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "NSA_IDX_INJECT needs idx");
  if (idx != nullptr && (reinterpret_cast<uintptr_t>(idx) & 3u) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "idx is not 4-byte aligned");
  if (workspace_bytes < pl.total)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.total, workspace_bytes);
  nsa::DsaArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = desc->batch;
  a.L = desc->seqlen;
  a.Hq = desc->n_q_heads;
  a.G = desc->n_kv_heads;
  a.Hg = a.Hq / a.G;
  a.D = desc->head_dim;
  a.Hi = desc->idx_heads;
  a.Di = desc->idx_dim;
  a.topk = params->top_k;
  a.waves = pl.waves;
  a.heads_per_wave = pl.heads_per_wave;
  a.parts = pl.parts;
  a.gpw = pl.gpw;
  a.wg_waves = pl.wg_waves;
  a.idx_tiles = (a.L + nsa::kIdxWaves * nsa::kIdxTPW - 1) / (nsa::kIdxWaves * nsa::kIdxTPW);
  a.topk_cache = pl.topk_cache;
  const float sc = params->softmax_scale > 0.f ? params->softmax_scale : 1.0f / std::sqrt(static_cast<float>(a.D));
  a.scale_log2 = sc * nsa::kLog2eHost;
  a.inject = inject ? 1 : 0;
  a.q = q;
  a.k = k;
  a.v = v;
  a.qi = qi;
  a.ki = ki;
  a.w = w;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.scores = reinterpret_cast<float*>(ws + pl.off_scores);
  a.idx = idx != nullptr ? idx : reinterpret_cast<int32_t*>(ws + pl.off_idx);
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = desc->q_stride[i];
    a.ks[i] = desc->k_stride[i];
    a.vs[i] = desc->v_stride[i];
    a.os[i] = desc->o_stride[i];
    a.qis[i] = desc->qi_stride[i];
  }
  for (int i = 0; i < 2; ++i) {
    a.kis[i] = desc->ki_stride[i];
    a.wis[i] = desc->w_stride[i];
  }
  hipError_t e = nsa::launch_dsa(a, desc->in_dtype == NSA_BF16, desc->out_dtype == NSA_BF16,
                                 static_cast<hipStream_t>(stream),
                                 reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "HIP error in the sparse attention launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

nsa_status_t nsa_dsa_workspace_bytes(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, size_t* bytes) {
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DsaPlan pl;
  NSA_TRY(plan_dsa(desc, params, &pl));
  *bytes = pl.total;
  return ok();
}

nsa_status_t nsa_dsa_prefill(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, const void* q,
                             const void* k, const void* v, const void* qi, const void* ki, const void* w, void* out,
                             int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return dsa_impl(desc, params, q, k, v, qi, ki, w, out, idx, idx_mode, workspace, workspace_bytes, stream, nullptr);
}

nsa_status_t nsa_dsa_prefill_timed(const nsa_dsa_desc_t* desc, const nsa_dsa_params_t* params, const void* q,
                                   const void* k, const void* v, const void* qi, const void* ki, const void* w,
                                   void* out, int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (stage_events == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events is NULL");
  for (int i = 0; i <= nsa::kDsaStages; ++i)
    if (stage_events[i] == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events[%d] is NULL", i);
  return dsa_impl(desc, params, q, k, v, qi, ki, w, out, idx, idx_mode, workspace, workspace_bytes, stream,
                  stage_events);
}

nsa_status_t nsa_fwd_prefill_timed(const nsa_prefill_desc_t* desc, const nsa_params_t* params,
                                   const void* q, const void* k, const void* v, const void* gates,
                                   void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* stage_events) {
  if (stage_events == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events is NULL");
  for (int i = 0; i <= nsa::kPrefillStages; ++i)
    if (stage_events[i] == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events[%d] is NULL", i);
  return prefill_impl(desc, params, 0, nullptr, nullptr, q, k, v, gates, out, idx, idx_mode, workspace,
                      workspace_bytes, stream, stage_events);
}

static nsa_status_t decode_impl(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                const void* q, const void* k_cache, const void* v_cache,
                                const void* kc_cache, const void* vc_cache, const int32_t* seqlens,
                                const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events, bool general = false, const nsa_general_t* gen = nullptr) {
  DecodePlan pl;
  Geometry geo;
  NSA_TRY(plan_decode(desc, params, &pl, general, gen, &geo));
  if (idx_mode != NSA_IDX_COMPUTE && idx_mode != NSA_IDX_INJECT)
    return fail(NSA_ERR_INVALID_ARGUMENT, "unknown idx_mode %d", static_cast<int>(idx_mode));
  if (desc->batch == 0) return ok();
  NSA_TRY(check_ptr("q", q, true));
  NSA_TRY(check_ptr("k_cache", k_cache, true));
  NSA_TRY(check_ptr("v_cache", v_cache, true));
  NSA_TRY(check_ptr("kc_cache", kc_cache, true));
  NSA_TRY(check_ptr("vc_cache", vc_cache, true));
  NSA_TRY(check_ptr("seqlens", seqlens, false));
  if (!geo.gate_layer()) NSA_TRY(check_ptr("gates", gates, false));
  NSA_TRY(check_ptr("out", out, false));
  NSA_TRY(check_ptr("workspace", workspace, true));
  if (idx_mode == NSA_IDX_INJECT && idx == nullptr)
    return fail(NSA_ERR_INVALID_ARGUMENT, "NSA_IDX_INJECT needs idx");
  if (idx != nullptr && (reinterpret_cast<uintptr_t>(idx) & 3u) != 0)
    return fail(NSA_ERR_INVALID_ARGUMENT, "idx is not 4-byte aligned");
  if (workspace_bytes < pl.total)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.total,
                workspace_bytes);
  nsa::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = desc->batch;
  a.Lmax = desc->max_seqlen;
  a.Nmax = desc->max_blocks;
  a.Hq = desc->n_q_heads;
  a.G = desc->n_kv_heads;
  a.Hg = a.Hq / a.G;
  a.D = desc->head_dim;
  a.n = params->select_top_k;
  a.w = params->sliding_window;
  a.NmaxPad = pl.NmaxPad;
  a.scale_log2 = scale_log2(params, a.D);
  a.inject = idx_mode == NSA_IDX_INJECT ? 1 : 0;
  a.q = q;
  a.kcache = k_cache;
  a.vcache = v_cache;
  a.kccache = kc_cache;
  a.vccache = vc_cache;
  a.seqlens = seqlens;
  a.gates = gates;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.logits_lds = pl.logits_lds ? 1 : 0;
  a.logits = reinterpret_cast<float*>(ws + pl.off_logits);
  a.idx = idx != nullptr ? idx : reinterpret_cast<int32_t*>(ws + pl.off_idx);
  a.gen = general ? 1 : 0;
  a.cl = params->compress_block_size;
  a.cd = geo.stride;
  a.ls = params->select_block_size;
  a.inv_cl = 1.0f / static_cast<float>(a.cl);
  if (geo.gate_layer()) {
    a.gate_w = gen->gate_w;
    a.gate_b = gen->gate_b;
    a.gates32 = reinterpret_cast<float*>(ws + pl.off_gates);
  }
  for (int i = 0; i < 2; ++i) {
    a.qs[i] = desc->q_stride[i];
    a.gs[i] = desc->g_stride[i];
    a.os[i] = desc->o_stride[i];
  }
  for (int i = 0; i < 3; ++i) {
    a.ks[i] = desc->k_stride[i];
    a.vs[i] = desc->v_stride[i];
    a.kcs[i] = desc->kc_stride[i];
    a.vcs[i] = desc->vc_stride[i];
  }
  hipError_t e = nsa::launch_decode(a, desc->in_dtype == NSA_BF16, desc->out_dtype == NSA_BF16,
                                    static_cast<hipStream_t>(stream),
                                    reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "HIP error in decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free decode

// Scratch of nsa_fwd_decode_noalloc: a file-scope device array, so that the
// call allocates nothing. Each GPU the library runs on holds its own copy
// (at its own address) until the process ends. In host code the array's name
// is only a stand-in; its device address is looked up per device with
// hipGetSymbolAddress and that address is what the kernels receive.
constexpr size_t kNoAllocScratchBytes = size_t{40} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on its first use on
// that device, with that device current).
nsa_status_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(NSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(NSA_ERR_HIP, "hipGetSymbolAddress of the decode scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return NSA_OK;
}
}  // namespace

extern "C" {

nsa_status_t nsa_fwd_decode_noalloc(const nsa_decode_desc_t* desc, const nsa_params_t* params, const void* q,
                                    const void* k_cache, const void* v_cache, const void* kc_cache,
                                    const void* vc_cache, const int32_t* seqlens, const void* gates, void* out,
                                    int32_t* idx, nsa_idx_mode_t idx_mode, void* stream) {
  DecodePlan pl;
  NSA_TRY(plan_decode(desc, params, &pl));
  if (pl.total > kNoAllocScratchBytes)
    return fail(NSA_ERR_WORKSPACE_TOO_SMALL,
                "this decode needs %zu bytes of scratch; the allocation-free decode holds %zu "
                "(use nsa_fwd_decode with a workspace)", pl.total, kNoAllocScratchBytes);
  if (desc->batch == 0)
    return decode_impl(desc, params, q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, out, idx, idx_mode,
                       nullptr, 0, stream, nullptr);
  void* ws = nullptr;
  NSA_TRY(noalloc_scratch(&ws));
  return decode_impl(desc, params, q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, out, idx, idx_mode, ws,
                     kNoAllocScratchBytes, stream, nullptr);
}

nsa_status_t nsa_fwd_decode(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                            const void* q, const void* k_cache, const void* v_cache,
                            const void* kc_cache, const void* vc_cache, const int32_t* seqlens,
                            const void* gates, void* out, int32_t* idx, nsa_idx_mode_t idx_mode,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(desc, params, q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, out, idx,
                     idx_mode, workspace, workspace_bytes, stream, nullptr);
}

nsa_status_t nsa_decode_general_workspace_bytes(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                                const nsa_general_t* general, size_t* bytes) {
  if (bytes == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  DecodePlan pl;
  NSA_TRY(plan_decode(desc, params, &pl, true, general));
  *bytes = pl.total;
  return ok();
}

nsa_status_t nsa_fwd_decode_general(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                    const nsa_general_t* general, const void* q, const void* k_cache,
                                    const void* v_cache, const void* kc_cache, const void* vc_cache,
                                    const int32_t* seqlens, const void* gates, void* out, int32_t* idx,
                                    nsa_idx_mode_t idx_mode, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return decode_impl(desc, params, q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, out, idx, idx_mode,
                     workspace, workspace_bytes, stream, nullptr, true, general);
}

nsa_status_t nsa_fwd_decode_timed(const nsa_decode_desc_t* desc, const nsa_params_t* params,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  const void* kc_cache, const void* vc_cache,
                                  const int32_t* seqlens, const void* gates, void* out,
                                  int32_t* idx, nsa_idx_mode_t idx_mode, void* workspace,
                                  size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (stage_events == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events is NULL");
  for (int i = 0; i <= nsa::kDecodeStages; ++i)
    if (stage_events[i] == nullptr) return fail(NSA_ERR_INVALID_ARGUMENT, "stage_events[%d] is NULL", i);
  return decode_impl(desc, params, q, k_cache, v_cache, kc_cache, vc_cache, seqlens, gates, out, idx,
                     idx_mode, workspace, workspace_bytes, stream, stage_events);
}

nsa_status_t nsa_compress_kv(int32_t batch, int32_t n_kv_heads, int32_t n_tokens, int32_t head_dim,
                             nsa_dtype_t dtype, int32_t block_size, const void* k,
                             const int64_t k_stride[3], const void* v, const int64_t v_stride[3],
                             void* kc, const int64_t kc_stride[3], void* vc,
                             const int64_t vc_stride[3], void* stream) {
  if (batch < 0 || n_kv_heads < 1 || n_tokens < 0 || head_dim < 1)
    return fail(NSA_ERR_INVALID_ARGUMENT, "batch, n_tokens >= 0 and n_kv_heads, head_dim >= 1 required");
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (block_size < 1) return fail(NSA_ERR_INVALID_ARGUMENT, "block_size must be >= 1");
  if (block_size != nsa::kBlock) return fail(NSA_ERR_UNSUPPORTED, "only block_size 64 is supported");
  if (head_dim > 1024) return fail(NSA_ERR_UNSUPPORTED, "head_dim > 1024 is not supported");
  if (k_stride == nullptr || v_stride == nullptr || kc_stride == nullptr || vc_stride == nullptr)
    return fail(NSA_ERR_INVALID_ARGUMENT, "stride array is NULL");
  NSA_TRY(check_strides("k", k_stride, 3, false));
  NSA_TRY(check_strides("v", v_stride, 3, false));
  NSA_TRY(check_strides("kc", kc_stride, 3, false));
  NSA_TRY(check_strides("vc", vc_stride, 3, false));
  const int nc = n_tokens / 64;
  if (batch == 0 || nc == 0) return ok();
  NSA_TRY(check_ptr("k", k, false));
  NSA_TRY(check_ptr("v", v, false));
  NSA_TRY(check_ptr("kc", kc, false));
  NSA_TRY(check_ptr("vc", vc, false));
  hipError_t e = nsa::launch_compress(batch, n_kv_heads, nc, head_dim, dtype == NSA_BF16, k, k_stride,
                                      v, v_stride, kc, kc_stride, vc, vc_stride,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "HIP error in compress launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
