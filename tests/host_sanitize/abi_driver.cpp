// Host-side check of the C ABI's argument validation under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Every call below must be rejected (or be a
// no-op) on the host before any HIP call, so no GPU is needed; extreme sizes
// exercise the overflow guards of the size arithmetic.  Exit status 0 when
// every return code is the expected one; a sanitizer report aborts the run.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "attn.h"

namespace {

int failures = 0;
int checks = 0;

void expect(const char* what, int got, int want) {
  ++checks;
  if (got != want) {
    ++failures;
    printf("FAIL %s: got %d (%s), want %d\n", what, got, attn_strerror(got), want);
  }
}

void expect_size(const char* what, size_t got, size_t want) {
  ++checks;
  if (got != want) {
    ++failures;
    printf("FAIL %s: got %zu, want %zu\n", what, got, want);
  }
}

// a non-null, 16-byte aligned address that is never dereferenced
void* const F = reinterpret_cast<void*>(0x10000);
void* const F2 = reinterpret_cast<void*>(0x10002);
const int32_t* const I = reinterpret_cast<const int32_t*>(0x10000);
const int32_t* const I2 = reinterpret_cast<const int32_t*>(0x10002);
float* const L = reinterpret_cast<float*>(0x10000);

int fwd(const void* q, void* o, int B, int H, int Hkv, int Sq, int Sk, int d, float scale, int dtype) {
  return attn_fwd(q, F, F, o, L, B, H, Hkv, Sq, Sk, d, 1, scale, dtype, nullptr);
}

int verify(int B, int H, int Hkv, int kq, int d, int maxs, int stride, size_t wsb, const int32_t* sl = I,
           void* ws = F) {
  return attn_verify(F, F, F, sl, maxs, stride, F, L, B, H, Hkv, kq, d, 0.088f, ATTN_BF16, ws, wsb, nullptr);
}

int paged(int B, int H, int Hkv, int kq, int page, int maxb, int npages, int maxs, size_t wsb,
          const int32_t* table = I) {
  return attn_verify_paged(F, F, F, table, maxb, npages, page, I, maxs, F, L, B, H, Hkv, kq, 128, 0.088f,
                           ATTN_BF16, F, wsb, nullptr);
}

}  // namespace

int main() {
  const int M = INT_MAX;
  // attn_fwd
  expect("fwd null q", fwd(nullptr, F, 1, 4, 2, 16, 16, 128, 0.1f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd misaligned q", fwd(F2, F, 1, 4, 2, 16, 16, 128, 0.1f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd H % Hkv", fwd(F, F, 1, 5, 2, 16, 16, 128, 0.1f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd scale 0", fwd(F, F, 1, 4, 2, 16, 16, 128, 0.f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd scale inf", fwd(F, F, 1, 4, 2, 16, 16, 128, 1.f / 0.f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd d 96", fwd(F, F, 1, 4, 2, 16, 16, 96, 0.1f, ATTN_BF16), ATTN_ERR_UNSUPPORTED);
  expect("fwd dtype 7", fwd(F, F, 1, 4, 2, 16, 16, 128, 0.1f, 7), ATTN_ERR_UNSUPPORTED);
  expect("fwd negative B", fwd(F, F, -1, 4, 2, 16, 16, 128, 0.1f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd INT_MIN Sq", fwd(F, F, 1, 4, 2, INT_MIN, 16, 128, 0.1f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd huge B*H*Sq", fwd(F, F, M, M, M, 1 << 30, 1 << 30, 128, 0.1f, ATTN_BF16), ATTN_ERR_INVALID_ARG);
  expect("fwd huge Sq (f32)", fwd(F, F, 1, 1, 1, M, 1, 128, 0.1f, ATTN_F32), ATTN_ERR_UNSUPPORTED);
  expect("fwd Sq 2^30 + 1", fwd(F, F, 1, 1, 1, (1 << 30) + 1, 1, 64, 0.1f, ATTN_BF16), ATTN_ERR_UNSUPPORTED);
  expect("fwd huge Sk", fwd(F, F, 1, 1, 1, 1, M, 128, 0.1f, ATTN_BF16), ATTN_ERR_UNSUPPORTED);
  expect("fwd 2^21 x 2^21 heads", fwd(F, F, 1 << 21, 1 << 21, 1, 1 << 21, 1, 64, 0.1f, ATTN_BF16),
         ATTN_ERR_INVALID_ARG);
  expect("fwd B = 0", fwd(nullptr, nullptr, 0, 4, 2, 16, 16, 128, 0.1f, ATTN_BF16), ATTN_OK);
  expect("fwd Sq = 0", fwd(nullptr, nullptr, 1, 4, 2, 0, 16, 128, 0.1f, ATTN_BF16), ATTN_OK);

  // attn_verify_workspace_bytes and attn_verify
  const size_t ws = attn_verify_workspace_bytes(8, 32, 8, 5, 128);
  expect("verify ws > 0", ws > 0 ? 0 : 1, 0);
  expect_size("verify ws huge", attn_verify_workspace_bytes(M, M, 1, M, 128), 0);
  expect_size("verify ws bad d", attn_verify_workspace_bytes(1, 8, 8, 5, 96), 0);
  expect_size("verify ws Hkv 3", attn_verify_workspace_bytes(1, 8, 3, 5, 128), 0);
  expect("verify ok-but-small ws", verify(8, 32, 8, 5, 128, 3000, 3000, ws - 1), ATTN_ERR_WORKSPACE);
  expect("verify null seqlens", verify(8, 32, 8, 5, 128, 3000, 3000, ws, nullptr), ATTN_ERR_INVALID_ARG);
  expect("verify misaligned seqlens", verify(8, 32, 8, 5, 128, 3000, 3000, ws, I2), ATTN_ERR_INVALID_ARG);
  expect("verify null ws", verify(8, 32, 8, 5, 128, 3000, 3000, ws, I, nullptr), ATTN_ERR_INVALID_ARG);
  expect("verify max > stride", verify(8, 32, 8, 5, 128, 3001, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("verify 68 packed rows", verify(8, 32, 8, 17, 128, 3000, 3000, ws), ATTN_ERR_UNSUPPORTED);
  expect("verify kq INT_MAX", verify(8, 32, 8, M, 128, 3000, 3000, ws), ATTN_ERR_UNSUPPORTED);
  expect("verify H INT_MAX", verify(1, M, 1, 1, 128, 3000, 3000, ws), ATTN_ERR_UNSUPPORTED);
  expect("verify total keys >= 2^31", verify(M, 8, 8, 1, 128, M, M, ws), ATTN_ERR_UNSUPPORTED);
  expect("verify huge cache", verify(1 << 16, 8, 8, 1, 128, 1 << 14, M, ws), ATTN_ERR_INVALID_ARG);
  expect("verify B = 0", attn_verify(nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr, 0, 32, 8, 5, 128,
                                     0.088f, ATTN_BF16, nullptr, 0, nullptr),
         ATTN_OK);
  // attn_verify_noalloc: the static scratch limit
  expect("noalloc too large", attn_verify_noalloc(F, F, F, I, 3000, 3000, F, L, 12, 32, 8, 5, 128, 0.088f, ATTN_BF16,
                                                  nullptr),
         ATTN_ERR_TOO_LARGE);
  expect("noalloc null q", attn_verify_noalloc(nullptr, F, F, I, 3000, 3000, F, L, 8, 32, 8, 5, 128, 0.088f,
                                               ATTN_BF16, nullptr),
         ATTN_ERR_INVALID_ARG);
  // attn_verify_tree
  expect("tree null mask", attn_verify_tree(F, F, F, I, 3000, 3000, nullptr, F, L, 8, 32, 8, 5, 128, 0.088f,
                                            ATTN_BF16, F, ws, nullptr),
         ATTN_ERR_INVALID_ARG);
  expect("tree 33 nodes", attn_verify_tree(F, F, F, I, 3000, 3000, reinterpret_cast<const uint32_t*>(F), F, L, 1, 8,
                                           8, 33, 128, 0.088f, ATTN_BF16, F, ~(size_t)0, nullptr),
         ATTN_ERR_UNSUPPORTED);

  // attn_verify_paged
  expect("paged page 8", paged(2, 32, 8, 5, 8, 100, 400, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("paged page 48", paged(2, 32, 8, 5, 48, 100, 400, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("paged page INT_MIN", paged(2, 32, 8, 5, INT_MIN, 100, 400, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("paged page INT_MAX", paged(2, 32, 8, 5, M, 100, 400, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("paged table too short", paged(2, 32, 8, 5, 64, 10, 400, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("paged huge table", paged(1 << 20, 32, 8, 1, 4096, 1 << 21, 400, 1, ws), ATTN_ERR_INVALID_ARG);
  expect("paged total keys >= 2^31", paged(M, 32, 8, 1, 4096, M, 400, M, ws), ATTN_ERR_UNSUPPORTED);
  expect("paged huge pool", paged(1, 32, 8, 1, 4096, 100, M, 3000, ws), ATTN_ERR_INVALID_ARG);
  expect("paged null table", paged(2, 32, 8, 5, 64, 100, 400, 3000, ws, nullptr), ATTN_ERR_INVALID_ARG);
  expect("paged small ws", paged(2, 32, 8, 5, 64, 100, 400, 3000, 100), ATTN_ERR_WORKSPACE);

  // attn_spec_accept
  const size_t sws = attn_spec_accept_workspace_bytes(8, 32000);
  expect_size("spec ws V too large", attn_spec_accept_workspace_bytes(8, (1 << 22) + 1), 0);
  expect("spec V too large", attn_spec_accept(I, L, L, L, L, const_cast<int32_t*>(I), const_cast<int32_t*>(I), 8, 5,
                                              (1 << 22) + 1, F, ~(size_t)0, nullptr),
         ATTN_ERR_UNSUPPORTED);
  expect("spec k INT_MAX", attn_spec_accept(I, L, L, L, L, const_cast<int32_t*>(I), const_cast<int32_t*>(I), M, M,
                                            1 << 22, F, ~(size_t)0, nullptr),
         ATTN_ERR_INVALID_ARG);
  expect("spec small ws", attn_spec_accept(I, L, L, L, L, const_cast<int32_t*>(I), const_cast<int32_t*>(I), 8, 5,
                                           32000, F, sws - 1, nullptr),
         ATTN_ERR_WORKSPACE);
  expect("spec B = 0", attn_spec_accept(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 5, 32000,
                                        nullptr, 0, nullptr),
         ATTN_OK);

  // attn_bwd
  const size_t bws = attn_bwd_workspace_bytes(2, 4, 100);
  expect_size("bwd ws huge", attn_bwd_workspace_bytes(M, M, M), 0);
  expect("bwd small ws", attn_bwd(F, F, F, F, F, L, F, F, F, 2, 4, 2, 100, 100, 128, 1, 0.1f, ATTN_BF16, F, bws - 1,
                                  nullptr),
         ATTN_ERR_WORKSPACE);
  expect("bwd huge", attn_bwd(F, F, F, F, F, L, F, F, F, M, M, 1, 1 << 30, 1 << 30, 128, 1, 0.1f, ATTN_BF16, F,
                              ~(size_t)0, nullptr),
         ATTN_ERR_INVALID_ARG);
  expect("bwd Sk 2^30 + 1", attn_bwd(F, F, F, F, F, L, F, F, F, 1, 1, 1, 1, (1 << 30) + 1, 64, 1, 0.1f, ATTN_BF16, F,
                                     ~(size_t)0, nullptr),
         ATTN_ERR_UNSUPPORTED);
  expect("bwd f32", attn_bwd(F, F, F, F, F, L, F, F, F, 2, 4, 2, 100, 100, 128, 1, 0.1f, ATTN_F32, F, bws, nullptr),
         ATTN_ERR_UNSUPPORTED);

  // attn_strerror
  for (int c = -6; c <= 1; ++c) expect("strerror non-null", attn_strerror(c) != nullptr ? 0 : 1, 0);

  printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
