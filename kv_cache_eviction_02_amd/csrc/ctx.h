// The library-owned context behind the opaque h2o_ctx of include/h2o.h, and
// the prefill steps shared by the C ABI's prefill entry points.
#pragma once

#include <stdint.h>

#include "h2o.h"
#include "launch.h"

struct h2o_ctx {
  h2o_config cfg;
  h2o_state st;
  int32_t k;
  int32_t waves;
  float scale_log2;
  int32_t t;        // absolute position of the next token to decode
  int32_t n_live;   // live slots per unit
  bool has_state;
  int32_t stride;   // scratch row stride (floats)
  float* scratch;   // 2 * units * stride floats: row log-sum-exp, column sums
  h2o::SplitScratch split;  // split decode scratch (split.splits < 2: unused)
  void* split_mem;
  int64_t multi_capacity;   // units the multi-step kernel keeps resident at once; -1 = not asked yet
  int32_t cus;              // compute units of the ctx's device; -1 = not asked yet
  int64_t lds_limit;        // LDS one workgroup may take on the ctx's device; -1 = not asked yet
};

namespace h2o {

// Argument checks common to the prefill entry points (pointers, alignment,
// 1 <= prompt_len <= H2O_MAX_PROMPT, grid size); the scratch capacity is the
// caller's to check.
h2o_status check_prefill(const h2o_ctx* ctx, const void* q, const void* k, const void* v, int32_t prompt_len,
                         const float* out);

// Enqueue the three prefill kernels with the given row statistics / column
// sum scratch (each units * stride floats, stride >= prompt_len) and, on
// success, set the ctx counters to the state after the prompt.
h2o_status run_prefill(h2o_ctx* ctx, const void* q, const void* k, const void* v, int32_t prompt_len, float* out,
                       float* row_lse, float* colsum, int32_t stride, void* stream);

}  // namespace h2o
