// Drives every C-ABI entry point through its argument validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host (the launchers are stubs that fail, so nothing
// reaches a device).  Fixed cases check the documented status; sweeps over extreme sizes,
// ranks and leading dimensions check that validation never overflows, reads out of bounds or
// returns a status outside the documented set.  Pointers are fake, 16-byte aligned addresses
// that are never dereferenced.  Exit status: the number of failed checks.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "tp_shard.h"

namespace {
int failures = 0;
long calls = 0;

void expect(const char* what, int got, int want) {
  ++calls;
  if (got != want) {
    ++failures;
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
  }
}
void valid_status(const char* what, long long got) {
  ++calls;
  if (got > 0 || got < TP_ERR_SCRATCH) {
    ++failures;
    std::printf("FAIL %s: status %lld outside the documented set\n", what, got);
  }
}

void* const P = (void*)(uintptr_t)0x100000;   // aligned, never dereferenced
void* const Q = (void*)(uintptr_t)0x100008;   // 8-byte aligned only
float* const F = (float*)P;
const int64_t BIG = INT64_MAX, HUGE = (int64_t)1 << 40;
const int64_t SIZES[] = {-1, 0, 1, 7, 8, 64, 4096, 12288, (int64_t)1 << 31, HUGE, BIG / 2, BIG};
const int RANKS[] = {-1, 0, 1, 7, 8};
const int WORLDS[] = {0, 1, 2, 8, 1 << 20};
}  // namespace

int main() {
  // ---- fixed cases (the documented status of each)
  expect("col null X", tp_col_linear_gelu(nullptr, P, P, 512, 64, 256, 1024, 0, 2, 0, TP_BF16, nullptr), TP_ERR_NULL);
  expect("col dtype", tp_col_linear_gelu(P, P, P, 512, 64, 256, 1024, 0, 2, 0, 7, nullptr), TP_ERR_DTYPE);
  expect("col rank", tp_col_linear_gelu(P, P, P, 512, 64, 256, 1024, 2, 2, 0, TP_BF16, nullptr), TP_ERR_RANK);
  expect("col N % world", tp_col_linear_gelu(P, P, P, 512, 64, 256, 1000, 0, 3, 0, TP_BF16, nullptr), TP_ERR_DIVISIBLE);
  expect("col align", tp_col_linear_gelu(Q, P, P, 512, 64, 256, 1024, 0, 2, 0, TP_BF16, nullptr), TP_ERR_ALIGN);
  expect("col valid -> launch", tp_col_linear_gelu(P, P, P, 512, 64, 256, 1024, 0, 2, 0, TP_BF16, nullptr), TP_ERR_LAUNCH);
  expect("row null", tp_row_linear_partial(P, 256, nullptr, F, 64, 1024, 256, 0, 2, TP_BF16, nullptr), TP_ERR_NULL);
  expect("row valid -> launch", tp_row_linear_partial(P, 1024, P, F, 64, 1024, 256, 1, 2, TP_BF16, nullptr), TP_ERR_LAUNCH);
  expect("attn workspace", tp_attn_head_shard(P, P, P, F, 2, 128, 1024, 8, 128, 0, 2, 1, TP_BF16, P, 16, nullptr), TP_ERR_WORKSPACE);
  const size_t ws = tp_attn_workspace_bytes(2, 128, 1024, 8, 128, 2, TP_BF16);
  expect("attn valid -> launch", tp_attn_head_shard(P, P, P, F, 2, 128, 1024, 8, 128, 0, 2, 1, TP_BF16, P, ws, nullptr), TP_ERR_LAUNCH);
  expect("attn noalloc beyond scratch", tp_attn_head_shard_noalloc(P, P, P, F, 8, 4096, 12288, 96, 128, 0, 8, 1, TP_BF16, nullptr), TP_ERR_SCRATCH);
  expect("reduce no input", tp_partial_reduce_residual_ln(nullptr, 0, 0, nullptr, nullptr, nullptr, 1e-5f, P, nullptr, 64, 256, TP_BF16, nullptr), TP_ERR_NULL);
  expect("reduce H % 8", tp_partial_reduce_residual_ln(F, 2, 64 * 260, P, P, P, 1e-5f, P, P, 64, 260, TP_BF16, nullptr), TP_ERR_ALIGN);
  expect("reduce valid -> launch", tp_partial_reduce_residual_ln(F, 2, 64 * 256, P, P, P, 1e-5f, P, P, 64, 256, TP_BF16, nullptr), TP_ERR_LAUNCH);
  expect("scatter rank", tp_partial_reduce_scatter_residual_ln(F, 2, 64 * 256, P, P, P, 1e-5f, P, P, 64, 256, 4, 4, TP_BF16, nullptr), TP_ERR_RANK);
  expect("row bf16 valid -> launch", tp_row_linear_partial_bf16(P, 1024, P, P, 64, 1024, 256, 1, 2, nullptr), TP_ERR_LAUNCH);
  expect("attn bf16 valid -> launch", tp_attn_head_shard_bf16(P, P, P, P, 2, 128, 1024, 8, 128, 0, 2, 1, P, ws, nullptr), TP_ERR_LAUNCH);
  expect("reduce bf16 stride % 8", tp_partial_reduce_residual_ln_bf16(P, 2, 64 * 256 + 4, P, P, P, 1e-5f, P, P, 64, 256, nullptr), TP_ERR_ALIGN);
  expect("col bwd bf16 valid -> launch", tp_col_linear_backward_bf16(P, P, P, 512, P, F, 512, 64, 256, 1024, 0, 2, 1, nullptr), TP_ERR_LAUNCH);
  expect("col bwd bf16 misaligned dX", tp_col_linear_backward_bf16(P, P, P, 512, (char*)P + 8, F, 512, 64, 256, 1024, 0, 2, 1, nullptr), TP_ERR_ALIGN);
  expect("reduce bf16 valid -> launch", tp_partial_reduce_residual_ln_bf16(P, 2, 64 * 256, P, P, P, 1e-5f, P, P, 64, 256, nullptr), TP_ERR_LAUNCH);
  for (int s = 1; s >= -12; --s) {
    const char* str = tp_status_string(s);
    ++calls;
    if (!str) { ++failures; std::printf("FAIL status string %d is null\n", s); }
  }

  // ---- sweeps: extreme sizes, ranks and leading dimensions
  for (int64_t a : SIZES)
    for (int64_t b : SIZES)
      for (int64_t c : SIZES)
        for (int r : RANKS)
          for (int w : WORLDS) {
            for (int dt : {TP_F32, TP_BF16}) {
              valid_status("col", tp_col_linear_gelu(P, P, P, c, a, b, c, r, w, 1, dt, nullptr));
              valid_status("row", tp_row_linear_partial(P, b, P, F, a, b, c, r, w, dt, nullptr));
              valid_status("fold", tp_row_linear_fold(P, b, P, F, a, b, c, r, w, r & 1, dt, nullptr));
              valid_status("col save", tp_col_linear_gelu_save(P, P, P, c, P, c, a, b, c, r, w, dt, nullptr));
              valid_status("row bwd", tp_row_linear_backward(P, P, P, c, P, c, P, c, F, c, a, b, c, r, w, 1, r & 1, dt, nullptr));
              valid_status("col bwd", tp_col_linear_backward(P, P, P, c, F, F, b, a, b, c, r, w, r & 1, dt, nullptr));
              valid_status("reduce", tp_partial_reduce_residual_ln(F, r + 1, c, P, P, P, 1e-5f, P, P, a, b, dt, nullptr));
              valid_status("scatter", tp_partial_reduce_scatter_residual_ln(F, r + 1, c, P, P, P, 1e-5f, P, P, a, b, r, w, dt, nullptr));
            }
            valid_status("row bf16", tp_row_linear_partial_bf16(P, b, P, P, a, b, c, r, w, nullptr));
            valid_status("col bwd bf16", tp_col_linear_backward_bf16(P, P, P, c, P, F, b, a, b, c, r, w, r & 1, nullptr));
            valid_status("reduce bf16", tp_partial_reduce_residual_ln_bf16(P, r + 1, c, P, P, P, 1e-5f, P, P, a, b, nullptr));
            valid_status("scatter bf16", tp_partial_reduce_scatter_residual_ln_bf16(P, r + 1, c, P, P, P, 1e-5f, P, P, a, b, r, w, nullptr));
          }
  for (int64_t bt : SIZES)
    for (int64_t sq : SIZES)
      for (int64_t h : SIZES)
        for (int nh : {-1, 0, 1, 8, 96, 1 << 30})
          for (int hd : {0, 64, 128, 1 << 30})
            for (int w : WORLDS) {
              const size_t need = tp_attn_workspace_bytes(bt, sq, h, nh, hd, w, TP_BF16);
              ++calls;
              for (int r : RANKS) {
                valid_status("attn", tp_attn_head_shard(P, P, P, F, bt, sq, h, nh, hd, r, w, r & 1, TP_BF16, P, need, nullptr));
                valid_status("attn fold", tp_attn_head_shard_fold(P, P, P, F, bt, sq, h, nh, hd, r, w, 1, r & 1, TP_BF16, P, need, nullptr));
                valid_status("attn noalloc", tp_attn_head_shard_noalloc(P, P, P, F, bt, sq, h, nh, hd, r, w, 1, TP_BF16, nullptr));
                valid_status("attn bf16", tp_attn_head_shard_bf16(P, P, P, P, bt, sq, h, nh, hd, r, w, 1, P, need, nullptr));
              }
            }
  std::printf("%ld checks, %d failures\n", calls, failures);
  return failures;
}
