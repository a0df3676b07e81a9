// C ABI of the attention library: argument validation and dispatch.
//
// Every check runs on the host before the first HIP call, so a rejected call
// has no side effect and the checks can be exercised without a GPU.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/attn.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// A pointer must be non-null and aligned unless its tensor is empty.
bool ptr_ok(const void* p, size_t elems) { return elems == 0 || (p != nullptr && aligned16(p)); }

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

constexpr size_t kMaxElems = (size_t)1 << 40;  // keeps every index product in 64-bit range
constexpr int kMaxSeq = 1 << 30;               // query/key counts: row indices plus a block fit int32

// Product of non-negative sizes, exact or saturated at SIZE_MAX: it never
// wraps, so an oversized request cannot pass a limit check.  Any zero factor
// gives 0.
size_t prod(std::initializer_list<long long> xs) {
  size_t p = 1;
  bool over = false;
  for (long long x : xs) {
    if (x == 0) return 0;
    over |= __builtin_mul_overflow(p, (size_t)x, &p);
  }
  return over ? SIZE_MAX : p;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Hkv, int Sq, int Sk, int d,
                        int causal, float scale, int dtype, void* stream) {
  if (B < 0 || Sq < 0 || Sk < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (Sq > kMaxSeq || Sk > kMaxSeq) return ATTN_ERR_UNSUPPORTED;
  const size_t nq = prod({B, H, Sq, d});
  const size_t nk = prod({B, Hkv, Sk, d});
  if (nq > kMaxElems || nk > kMaxElems) return ATTN_ERR_INVALID_ARG;
  // one workgroup per (batch, head, query block) must fit the grid: blocks
  // of 256 rows (bf16) or 16 rows (fp32)
  const long long rows_per_block = dtype == ATTN_F32 ? 16 : 256;
  if (prod({B, H, ((long long)Sq + rows_per_block - 1) / rows_per_block}) > 0x7fffffffu)
    return ATTN_ERR_INVALID_ARG;
  if (!ptr_ok(q, nq) || !ptr_ok(o, nq) || !ptr_ok(k, nk) || !ptr_ok(v, nk)) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned4(lse)) return ATTN_ERR_INVALID_ARG;
  if (nq == 0) return ATTN_OK;

  attn::FwdArgs a{};  // every field zero/null until set
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == ATTN_BF16 ? attn::launch_fwd_bf16(a, s) : attn::launch_fwd_f32(a, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_verify_workspace_bytes(int B, int H, int Hkv, int kq, int d) {
  if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || kq < 1 || (d != 64 && d != 128)) return 0;
  if (prod({B, H, kq, d}) > kMaxElems) return 0;  // larger than any call accepts
  return attn::verify_workspace_bytes(B, H, Hkv, kq, d);
}

namespace {

int verify_contiguous(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                      int max_seqlen_k, int cache_stride, const uint32_t* tree_mask, bool tree, void* o,
                      float* lse, int B, int H, int Hkv, int kq, int d, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
  if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || kq < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_k < 0 || cache_stride < 0 || max_seqlen_k > cache_stride) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)(H / Hkv) * kq > 64) return ATTN_ERR_UNSUPPORTED;  // two 32-row query tiles at most
  if (tree && kq > 32) return ATTN_ERR_UNSUPPORTED;                  // 32-bit visibility masks
  if ((long long)B * max_seqlen_k >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;  // total keys fit int32
  const size_t nq = prod({B, H, kq, d});
  const size_t nk = prod({B, Hkv, cache_stride, d});
  if (nq > kMaxElems || nk > kMaxElems) return ATTN_ERR_INVALID_ARG;
  if (!ptr_ok(q, nq) || !ptr_ok(o, nq) || !ptr_ok(k_cache, nk) || !ptr_ok(v_cache, nk))
    return ATTN_ERR_INVALID_ARG;
  if (B > 0 && (seqlens_k == nullptr || !aligned4(seqlens_k))) return ATTN_ERR_INVALID_ARG;
  if (tree && B > 0 && (tree_mask == nullptr || !aligned4(tree_mask))) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned4(lse)) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::verify_workspace_bytes(B, H, Hkv, kq, d);
  if (noalloc) {
    if (need > attn::verify_noalloc_scratch_bytes()) return ATTN_ERR_TOO_LARGE;
  } else {
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (need > 0 && (workspace == nullptr || !aligned16(workspace))) return ATTN_ERR_INVALID_ARG;
  }
  if (nq == 0) return ATTN_OK;

  attn::VerifyArgs a{};  // every field zero/null until set
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens_k;
  a.paged = false;
  a.block_table = nullptr;
  a.max_blocks = 0;
  a.num_pages = 0;
  a.page_shift = 0;
  a.tree_mask = tree ? tree_mask : nullptr;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.kq = kq;
  a.d = d;
  a.max_seqlen_k = max_seqlen_k;
  a.cache_stride = cache_stride;
  a.scale = scale;
  a.workspace = workspace;
  const hipError_t e = noalloc ? attn::launch_verify_bf16_noalloc(a, static_cast<hipStream_t>(stream))
                               : attn::launch_verify_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" int attn_verify(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seqlens_k, int max_seqlen_k, int cache_stride,
                           void* o, float* lse, int B, int H, int Hkv, int kq, int d,
                           float scale, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return verify_contiguous(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, nullptr, false, o, lse,
                           B, H, Hkv, kq, d, scale, dtype, workspace, workspace_bytes, stream);
}

extern "C" int attn_verify_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* seqlens_k, int max_seqlen_k, int cache_stride,
                                   void* o, float* lse, int B, int H, int Hkv, int kq, int d,
                                   float scale, int dtype, void* stream) {
  return verify_contiguous(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, nullptr, false, o, lse,
                           B, H, Hkv, kq, d, scale, dtype, nullptr, 0, stream, true);
}

extern "C" int attn_verify_tree(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seqlens_k, int max_seqlen_k, int cache_stride,
                                const uint32_t* tree_mask, void* o, float* lse, int B, int H, int Hkv,
                                int kq, int d, float scale, int dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return verify_contiguous(q, k_cache, v_cache, seqlens_k, max_seqlen_k, cache_stride, tree_mask, true, o, lse,
                           B, H, Hkv, kq, d, scale, dtype, workspace, workspace_bytes, stream);
}

extern "C" int attn_verify_paged(const void* q, const void* k_pages, const void* v_pages,
                                 const int32_t* block_table, int max_blocks_per_seq, int num_pages,
                                 int page_size, const int32_t* seqlens_k, int max_seqlen_k,
                                 void* o, float* lse, int B, int H, int Hkv, int kq, int d,
                                 float scale, int dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || kq < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_k < 0 || max_blocks_per_seq < 0 || num_pages < 0) return ATTN_ERR_INVALID_ARG;
  int page_shift = 0;
  while (page_shift < 13 && (1 << page_shift) != page_size) ++page_shift;
  if (page_size < 16 || page_size > 4096 || (1 << page_shift) != page_size) return ATTN_ERR_INVALID_ARG;
  if ((long long)max_seqlen_k > (long long)max_blocks_per_seq * page_size) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)(H / Hkv) * kq > 64) return ATTN_ERR_UNSUPPORTED;  // two 32-row query tiles at most
  if ((long long)B * max_seqlen_k >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;  // total keys fit int32
  const size_t nq = prod({B, H, kq, d});
  const size_t nk = prod({num_pages, Hkv, page_size, d});
  const size_t nt = prod({B, max_blocks_per_seq});
  if (nq > kMaxElems || nk > kMaxElems || nt > kMaxElems) return ATTN_ERR_INVALID_ARG;
  if (!ptr_ok(q, nq) || !ptr_ok(o, nq) || !ptr_ok(k_pages, nk) || !ptr_ok(v_pages, nk))
    return ATTN_ERR_INVALID_ARG;
  if (B > 0 && (seqlens_k == nullptr || !aligned4(seqlens_k))) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_k > 0 && (block_table == nullptr || !aligned4(block_table))) return ATTN_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned4(lse)) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::verify_workspace_bytes(B, H, Hkv, kq, d);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (need > 0 && (workspace == nullptr || !aligned16(workspace))) return ATTN_ERR_INVALID_ARG;
  if (nq == 0) return ATTN_OK;

  attn::VerifyArgs a{};  // every field zero/null until set
  a.q = q;
  a.k = k_pages;
  a.v = v_pages;
  a.seqlens = seqlens_k;
  a.paged = true;
  a.block_table = block_table;
  a.tree_mask = nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.page_shift = page_shift;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.kq = kq;
  a.d = d;
  a.max_seqlen_k = max_seqlen_k;
  a.cache_stride = 0;
  a.scale = scale;
  a.workspace = workspace;
  const hipError_t e = attn::launch_verify_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_spec_accept_workspace_bytes(int B, int V) {
  if (B < 0 || V < 1 || V > (1 << 22)) return 0;
  return attn::spec_accept_workspace_bytes(B, V);
}

extern "C" int attn_spec_accept(const int32_t* draft_tokens, const float* draft_probs,
                                const float* target_probs, const float* u_accept,
                                const float* u_sample, int32_t* n_accepted, int32_t* out_tokens,
                                int B, int k, int V, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (B < 0 || k < 0 || V < 1) return ATTN_ERR_INVALID_ARG;
  if (V > (1 << 22)) return ATTN_ERR_UNSUPPORTED;  // fixed-point sums stay below 2^62
  if (prod({B, (long long)k + 1, V}) > kMaxElems) return ATTN_ERR_INVALID_ARG;
  if (B == 0) return ATTN_OK;
  const size_t nq = prod({B, k, V});
  if (k > 0 && (draft_tokens == nullptr || !aligned4(draft_tokens) || u_accept == nullptr ||
                !aligned4(u_accept) || nq == 0 || draft_probs == nullptr || !aligned4(draft_probs)))
    return ATTN_ERR_INVALID_ARG;
  if (target_probs == nullptr || !aligned4(target_probs) || u_sample == nullptr || !aligned4(u_sample) ||
      n_accepted == nullptr || !aligned4(n_accepted) || out_tokens == nullptr || !aligned4(out_tokens))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::spec_accept_workspace_bytes(B, V);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return ATTN_ERR_INVALID_ARG;
  attn::SpecAcceptArgs a{};  // every field zero/null until set
  a.draft_tokens = draft_tokens;
  a.draft_probs = draft_probs;
  a.target_probs = target_probs;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.n_accepted = n_accepted;
  a.out_tokens = out_tokens;
  a.B = B;
  a.k = k;
  a.V = V;
  a.workspace = workspace;
  const hipError_t e = attn::launch_spec_accept(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_bwd_workspace_bytes(int B, int H, int Sq) {
  if (B < 0 || H < 1 || Sq < 0) return 0;
  if (prod({B, H, Sq}) > kMaxElems) return 0;  // larger than any call accepts
  return attn::bwd_workspace_bytes(B, H, Sq);
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Sq,
                        int Sk, int d, int causal, float scale, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (B < 0 || Sq < 0 || Sk < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (Sq > kMaxSeq || Sk > kMaxSeq) return ATTN_ERR_UNSUPPORTED;
  const size_t nq = prod({B, H, Sq, d});
  const size_t nk = prod({B, Hkv, Sk, d});
  if (nq > kMaxElems || nk > kMaxElems) return ATTN_ERR_INVALID_ARG;
  if (prod({B, H, ((long long)Sq + 127) / 128}) > 0x7fffffffu) return ATTN_ERR_INVALID_ARG;
  if (!ptr_ok(q, nq) || !ptr_ok(o, nq) || !ptr_ok(dout, nq) || !ptr_ok(dq, nq)) return ATTN_ERR_INVALID_ARG;
  if (!ptr_ok(k, nk) || !ptr_ok(v, nk) || !ptr_ok(dk, nk) || !ptr_ok(dv, nk)) return ATTN_ERR_INVALID_ARG;
  if (nq > 0 && (lse == nullptr || !aligned4(lse))) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::bwd_workspace_bytes(B, H, Sq);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (need > 0 && (workspace == nullptr || !aligned16(workspace))) return ATTN_ERR_INVALID_ARG;
  if (nq == 0 && nk == 0) return ATTN_OK;
  attn::BwdArgs a{};  // every field zero/null until set
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.workspace = workspace;
  const hipError_t e = attn::launch_bwd_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer, size, or scale)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration (head dim, dtype, or query packing)";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP kernel launch failed";
    case ATTN_ERR_TOO_LARGE: return "sizes need more than the static scratch of attn_verify_noalloc (32 MiB)";
    default: return "unknown error code";
  }
}
