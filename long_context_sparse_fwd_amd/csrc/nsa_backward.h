// Internal interface of the prefill backward pass between the host API
// (nsa_api.cpp) and its kernels (nsa_backward.hip). Not installed, not part
// of the ABI.
#pragma once

#include "nsa_internal.h"

namespace nsa {

// Backward pass of the prefill (gradients for a fixed selection).
constexpr int kBwdSelPiece = 256;  // tokens per workgroup of the selected branch's key side
constexpr int kBwdCmpPiece = 512;  // tokens per workgroup of the compressed branch's key side
constexpr int kBwdStage = 2;      // tokens staged in LDS at a time by the key-side kernel (even)
struct BwdArgs {
  int B, L, Hq, G, Hg, D, n, w;
  int Nb, Nc, NcT;
  float scale_log2, scale;  // softmax scale * log2(e), softmax scale
  // workgroups per (sequence, group) of the key-side kernel, per branch
  // (compressed, selected, window)
  int bkv_units[3];
  const void* q;
  const void* k;
  const void* v;
  const void* gates;
  const void* dout;  // [B, L, Hq, D] in the output type
  const int32_t* idx;
  // Optional: the selected branch's output [B, L, Hq, D] (output type) and
  // natural-log log-sum-exp [B, L, Hq] saved by the forward; when given, the
  // query side takes them instead of recomputing that branch's forward.
  const void* o_slc;
  const float* lse_slc;
  float* dq;      // [B, L, Hq, D]
  float* dk;      // [B, L, G, D]
  float* dv;      // [B, L, G, D]
  float* dgates;  // [B, L, Hq, 3]
  int64_t qs[3], ks[3], vs[3], gs[3], os[3];
  // workspace
  void *ka, *kv, *va, *vv;      // [B][G][Nb] 64-key tiles: K, K^T-layout, V, V^T-layout
  void *kcm, *vcm;              // [B][Nc][G][D] block means
  void *kca, *kcv, *vca, *vcv;  // [B][G][NcT] the same four tile layouts of the block means
  void *qT, *dT;                // [B][L][G][D][16] head-minor q and dout (input type)
  void* dN;                     // [B][L][Hq][D] dout in the input type
  float2* stat;                 // [B][L][Hq][3] (log2-domain log-sum-exp, dout . o) per branch
  float *dkc, *dvc;             // [B][Nc][G][D] gradients of the block means
  int32_t* cnt;                 // [B][G][Nb] tokens per selected block (then fill cursors)
  int32_t* offs;                // [B][G][Nb + 1] list offsets
  int32_t* pofs;                // [B][G][Nb + 1] piece offsets
  int32_t* list;                // [B][G][L * n] tokens per selected block
};
constexpr int kBwdStages = 3;  // prep, query side, key side
hipError_t launch_backward(const BwdArgs& a, bool in_bf16, bool out_bf16, hipStream_t st, hipEvent_t* ev);


}  // namespace nsa
