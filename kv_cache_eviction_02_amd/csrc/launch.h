// Internal launch interface between the C ABI (h2o_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

struct DecodeArgs {
  const void* q;       // [U, d]
  const void* k_new;   // [U, d]
  const void* v_new;   // [U, d]
  void* k_slots;       // [U, k, d]
  void* v_slots;       // [U, k, d]
  float* score;        // [U, k]
  int32_t* pos;        // [U, k]
  float* k_scale;      // [U, k] E4M3 row scales (E4M3 cache only)
  float* v_scale;      // [U, k]
  float* out;          // [U, d]
  int32_t* evicted;    // [U] or null
  int32_t units;
  int32_t k, r;
  int32_t t;           // absolute position of the token being decoded
  int32_t n_ring;      // live ring slots: min(t, r)
  int32_t n_heavy;     // live heavy slots
  float scale_log2;    // softmax scale * log2(e)
  int32_t policy;      // 0 H2O, 1 static (victim = position leaving the window), 2 naive (no accumulation)
};

// Scratch of the split decode (several workgroups per unit).
struct SplitScratch {
  float* partials;     // [U, S, d + 2]: max, sum, output of each workgroup's rows
  float* logits;       // [U, k + 1]
  unsigned* counters;  // [U]: arrivals in the current step, zero between launches
  int32_t splits;      // S >= 2
};

struct PrefillArgs {
  const void* pq;      // prompt queries [U, P, d]
  const void* pk;      // prompt keys    [U, P, d]
  const void* pv;      // prompt values  [U, P, d]
  void* k_slots;
  void* v_slots;
  float* score;
  int32_t* pos;
  float* k_scale;      // E4M3 cache only
  float* v_scale;
  float* row_lse;      // scratch [U, stride]: per query row, log2 of the softmax denominator (log2 domain)
  float* colsum;       // scratch [U, stride]: accumulated attention per prompt position
  float* out;          // [U, P, d] float32 prompt attention output, or null
  int32_t units;
  int32_t stride;      // scratch row stride in floats: max_prompt rounded up to 16
  int32_t P;
  int32_t k, r, h;
  float scale_log2;
  int32_t last_row_only;  // scores = attention of the last prompt row (naive policy), not column sums
};

// dtype: 0 = float32, 1 = bfloat16 (inputs); cache: 0 = slots in the input
// dtype, 1 = E4M3 codes with per-row scales (bf16 inputs only).  Return
// hipSuccess or the launch error.
// sp == nullptr or sp->splits < 2: one workgroup per unit.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int cache, int head_dim, int waves,
                         const SplitScratch* sp, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int cache, int head_dim, hipStream_t s);

// n_steps consecutive steps in one launch (one workgroup per unit, no split):
// `a` describes the first step, live0 = live slots before it; inputs and
// outputs of step s start s * units rows further.  Requires
// decode_multi_fits(a.k, ...); with `resident` the unit's rows stay in LDS
// (decode_resident_lds bytes per workgroup, one workgroup per compute unit).
hipError_t launch_decode_multi(const DecodeArgs& a, int dtype, int cache, int head_dim, int waves, int n_steps,
                               int live0, bool resident, hipStream_t s);
// Static plus dynamic LDS of the resident multi-step kernel.
size_t decode_resident_lds(int k, int dtype, int cache, int head_dim, int waves);

// LDS a workgroup may take without opting in to more.
constexpr size_t kMaxLds = 64 * 1024;
// Static LDS of the decode kernels for this instantiation; the single-step
// kernels add (live slots + 1) * 4 bytes, the multi-step kernel (3k + 1) * 4.
size_t decode_static_lds(int dtype, int cache, int head_dim, int waves);
bool decode_multi_fits(int k, int dtype, int cache, int head_dim, int waves);
// Workgroups of the multi-step kernel one compute unit of the current device
// holds at once (registers, LDS, waves); 0 when it does not fit or the query fails.
int decode_multi_per_cu(int k, int dtype, int cache, int head_dim, int waves);

// Automatic wavefronts per unit for the decode kernel.
int decode_waves_auto(int units);
// Automatic workgroups per unit (1 = no split).
int decode_split_auto(int units, int waves, int k, int cus);

}  // namespace h2o
