// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, H, Hkv, Sq, Sk, d;
  int causal;
  float scale;
};

struct VerifyArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seqlens;
  bool paged;                  // false: contiguous cache [B][Hkv][cache_stride][d]
  const int32_t* block_table;  // paged: [B][max_blocks], pages [num_pages][Hkv][2^page_shift][d]
  int max_blocks, num_pages, page_shift;
  const uint32_t* tree_mask;   // [B][kq] visibility bitmasks among the new tokens; null: causal chain
  void* o;
  float* lse;  // may be null
  int B, H, Hkv, kq, d;
  int max_seqlen_k, cache_stride;
  float scale;
  void* workspace;
};

struct SpecAcceptArgs {
  const int32_t* draft_tokens;  // [B][k]
  const float* draft_probs;     // [B][k][V]
  const float* target_probs;    // [B][k+1][V]
  const float* u_accept;        // [B][k]
  const float* u_sample;        // [B]
  int32_t* n_accepted;          // [B]
  int32_t* out_tokens;          // [B][k+1]
  int B, k, V;
  void* workspace;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, Hkv, Sq, Sk, d;
  int causal;
  float scale;
  void* workspace;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_verify_bf16(const VerifyArgs& a, hipStream_t s);
// attn_verify with the library's static per-device scratch as the workspace
// (a.workspace is ignored); sizes must fit verify_noalloc_scratch_bytes().
hipError_t launch_verify_bf16_noalloc(const VerifyArgs& a, hipStream_t s);
size_t verify_noalloc_scratch_bytes();
hipError_t launch_spec_accept(const SpecAcceptArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);

// Workgroups of the verify split kernel and the workspace it needs.
int verify_split_workgroups();
size_t verify_workspace_bytes(int B, int H, int Hkv, int kq, int d);
size_t spec_accept_workspace_bytes(int B, int V);
size_t bwd_workspace_bytes(int B, int H, int Sq);

}  // namespace attn
