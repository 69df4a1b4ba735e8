// Internal interface between the host API (nsa_api.cpp) and the kernel
// launchers (*.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

constexpr int kBlock = 64;         // compress / select block size supported
constexpr int kSurvCap = 256;      // top-k survivor buffer per wave (entries)
constexpr int kCmpTPW = 2;         // tokens per wave, window+compressed+selection kernel
constexpr int kSelTPW = 2;         // tokens per wave, selected-branch kernel (4 waves)
constexpr int kSelRing = 2;        // half-block register buffers per wave in that kernel
constexpr int kMaxLds = 160 * 1024;
constexpr size_t kSelLdsOneWg = 81 * 1024;  // k_sel LDS (static + dynamic) for one workgroup per CU
constexpr float kLog2eHost = 1.4426950408889634f;

// Everything a prefill launch needs; passed by value to every kernel.
struct PrefillArgs {
  int B, L, Hq, G, Hg, D, n, w;
  int t0, Lq;  // the queries are positions [t0, t0 + Lq) = [t0, L) of the L-token context
  // Per-sequence lengths and first query positions (device arrays, or null
  // for L and t0 above). Sequence b then has a seq_lens[b]-token context and
  // query positions [q_offs[b], min(seq_lens[b], q_offs[b] + Lq)); Lq is the
  // number of query rows the q / gates / out / idx arrays hold.
  const int32_t* seq_lens;
  const int32_t* q_offs;
  int sel_interleave;  // k_sel's XCD mapping: 1 = a group's XCDs take its tiles in turn, 0 = contiguous
  // Contiguous mapping with G dividing 8: the XCDs of a group (8 / G of
  // them) take the (sequence, tile) items [sel_bounds[k], sel_bounds[k+1])
  // of the group; sel_bounds[0] = -1 selects the plain eighths instead.
  int sel_bounds[9];
  int Nb;   // 64-token key tiles = ceil(L / 64)
  int Nc;   // compressed blocks (wholly inside the context) = (L - cl) / cd + 1, or 0
  int NcT;  // 64-row chunks of the compressed tiles = ceil(Nc / 64)
  // Geometry: compressed block i covers tokens [i*cd, i*cd + cl); selection
  // blocks hold ls tokens (a multiple of 32). The plain geometry is
  // cl = cd = ls = 64 with block means.
  int cl, cd, ls;
  float inv_cl;   // 1 / cl
  int sel_map;    // 1: selection-block scores from the compressed scores by token overlap
  int cmp_in_prep;  // 1: k_prep writes the compressed tiles (means of its 64-token blocks)
  // Learned compressor (null: block means): w [D][cl][D] (output dim,
  // position in the block, input dim) and bias [D], in the input type.
  const void* wk;
  const void* bk;
  const void* wv;
  const void* bv;
  // Gate layer (null: the gates are given): gates = sigmoid(q . gate_w[h] +
  // gate_b[h]), gate_w [Hq][D][3], gate_b [Hq][3] in the input type, written
  // by k_gate as fp32 [B][Lq][Hq][3] into gates32, which the branches read.
  const void* gate_w;
  const void* gate_b;
  float* gates32;
  int cmp_waves, cmp_tiles, sel_tiles;
  int cmp_lo_lds;  // compressed kernel stages the low parts of the K means in LDS (8 waves only)
  int sel_bm_words;  // words of a k_sel wave's half-block bitmap (one byte per half block)
  int sel_pf;        // k_sel prefetches the rows its epilogue adds to into LDS (1) or reads them at the end (0)
  float scale_log2;  // softmax scale * log2(e)
  int inject;        // 1: idx holds the selection; 0: compute it into idx
  const void* q;
  const void* k;
  const void* v;
  const void* gates;
  void* out;
  int32_t* idx;
  void* kt;   // [B][G][Nb] 64-key K tiles (fragment-major)
  void* vt;   // [B][G][Nb] 64-key V^T tiles
  // bf16 output: the window + compressed part of each output row in fp32,
  // [B][Lq][Hq][D], which k_sel completes and rounds to bf16 once; null for
  // fp32 output (out itself holds that part until k_sel adds to it).
  float* part;
  void* kct;   // [B][G][NcT] 64-block tiles of block means of K times scale_log2 (bf16: the high part)
  void* kclt;  // bf16 input only: the low part, bf16(mean - high), same layout
  void* vct;   // [B][G][NcT] 64-block V^T tiles of block means of V
  int64_t qs[3], ks[3], vs[3], gs[3], os[3];
  // Optional (null: not written): the selected branch's own output
  // [B][Lq][Hq][D] in the output type and its natural-log log-sum-exp
  // [B][Lq][Hq] (-inf for no usable block), for the backward pass.
  void* save_o;
  float* save_lse;
  // Compressed kernel: each token's block-score row in the workspace,
  // [B][G][Lq + 2][NcT * 64] (two spare rows for the tokens past the last
  // query row), when the rows of 8 waves do not fit LDS; null: in LDS.
  float* cmp_sc;
};

struct DecodeArgs {
  int B, Lmax, Nmax, Hq, G, Hg, D, n, w;
  int NmaxPad;  // row length of the logits workspace: ceil(Lmax / 64) rounded up to 64
  float scale_log2;
  int inject;
  const void* q;
  const void* kcache;
  const void* vcache;
  const void* kccache;
  const void* vccache;
  const int32_t* seqlens;
  const void* gates;
  void* out;
  int32_t* idx;
  int logits_lds;  // 1: the compressed logits stay in LDS; 0: in `logits`
  float* logits;   // compressed logits (log2 domain), [B*G][16][NmaxPad], if !logits_lds
  int64_t qs[2], ks[3], vs[3], kcs[3], vcs[3], gs[2], os[2];
  // General geometry (gen = 1): compressed block i covers tokens [i*cd,
  // i*cd + cl) and is visible once i*cd + cl - 1 <= t; selection blocks hold
  // ls tokens, scored by the compressed-attention mass on their tokens. With
  // a gate layer (gate_w, gate_b: [Hq][D][3], [Hq][3] in the input type),
  // k_dgate writes the fp32 gates [B][Hq][3] into gates32 and the decode
  // reads those instead of `gates`.
  int gen, cl, cd, ls;
  float inv_cl;
  const void* gate_w;
  const void* gate_b;
  float* gates32;
};

// ev (nullable): kPrefillStages+1 / kDecodeStages+1 events recorded on st
// before each kernel and after the last one.
constexpr int kPrefillStages = 3;
constexpr int kDecodeStages = 1;
hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, bool out_bf16, hipStream_t st,
                          hipEvent_t* ev);
hipError_t launch_decode(const DecodeArgs& a, bool in_bf16, bool out_bf16, hipStream_t st,
                         hipEvent_t* ev);
hipError_t launch_compress(int B, int G, int Nc, int D, bool bf16, const void* k, const int64_t* ks,
                           const void* v, const int64_t* vs, void* kc, const int64_t* kcs,
                           void* vc, const int64_t* vcs, hipStream_t st);

// LDS bytes of the decode kernel, with or without room for the logits.
size_t dec_lds_bytes(int NmaxPad, int D, bool bf16, bool logits_lds);

size_t cmpwin_lds_bytes(int waves, int NcT, int D, bool bf16, bool lo_lds);

// Largest select_top_k * select_block_size: a k_sel wave's step list holds
// kSelTPW * 128 half blocks.
constexpr int kMaxSelTokens = 64 * 64;

// k_sel: bitmap words per wave (one byte per half block of Nb blocks, padded
// to 16 bytes) and the dynamic LDS of a launch.
inline int sel_bm_words(int Nb) { return (2 * Nb + 15) / 16 * 4; }
// k_sel's prefetch region: per wave the fp32 rows (kSelTPW tokens x 16 heads
// x D) that its epilogue adds the selected branch to
inline size_t sel_pf_bytes(int D) { return 4 * static_cast<size_t>(kSelTPW) * 16 * D * sizeof(float); }
size_t sel_lds_bytes(int Nb, int D, bool bf16, bool prefetch);
// static LDS of k_sel (query fragments of 4 waves)
inline size_t sel_static_lds_bytes(int D, bool bf16) {
  return 4 * static_cast<size_t>(kSelTPW) * (D / 32) * (bf16 ? 16 : 32) * 64;
}

// LDS bytes of the block scores of the compressed kernel, and its per-wave
// top-k scratch (which reuses the tile stage once the compressed passes end).
inline size_t cmp_lds_bytes(int waves, int NcT) {
  return static_cast<size_t>(waves) * kCmpTPW * NcT * 64 * sizeof(float);
}
inline size_t cmp_topk_scratch_bytes() { return kSurvCap * sizeof(uint64_t) + 64 * sizeof(int); }

}  // namespace nsa

namespace nsa {

// Token-level sparse attention with a ReLU indexer (DSA): the arguments of
// its three kernels.
struct DsaArgs {
  int B, L, Hq, G, Hg, D, Hi, Di, topk;
  int waves;        // attention waves per query token: 16 query heads each
  int heads_per_wave;  // min(Hg, 16)
  int parts;        // attention workgroups per query token (each takes gpw KV heads)
  int gpw;          // KV heads staged per attention workgroup
  int wg_waves;     // waves per attention workgroup
  int idx_tiles;    // indexer workgroups per sequence (kIdxWaves * kIdxTPW query tokens each)
  int topk_cache;   // orderable keys of a row kept in LDS by the top-k kernel
  float scale_log2; // softmax scale * log2(e)
  int inject;       // 1: idx holds the selection (a set of tokens)
  const void* q;
  const void* k;
  const void* v;
  const void* qi;
  const void* ki;
  const void* w;
  void* out;
  int32_t* idx;     // [B][L][topk], ascending, -1 padded
  float* scores;    // indexer scores, row t of sequence b at b*L(L+1)/2 + t(t+1)/2
  int64_t qs[3], ks[3], vs[3], os[3], qis[3], kis[2], wis[2];
};
constexpr int kIdxWaves = 8, kIdxTPW = 2;   // indexer: waves per workgroup, query tokens per wave
constexpr int kDsaStages = 3;
constexpr int kDsaMaxTopK = 2048;
hipError_t launch_dsa(const DsaArgs& a, bool in_bf16, bool out_bf16, hipStream_t st, hipEvent_t* ev);
size_t dsa_topk_lds_bytes(int cache);
size_t dsa_attn_lds_bytes(int groups_per_wg, int D, bool bf16, int k);

}  // namespace nsa
