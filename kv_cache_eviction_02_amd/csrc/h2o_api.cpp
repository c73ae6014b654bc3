// C ABI of the H2O hot path: argument validation, host-side position counters,
// prefill scratch ownership, and kernel launches.  Declarations and the full
// contract are in include/h2o.h.
#include "h2o.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <new>

#include "ctx.h"
#include "launch.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool valid_dims(const h2o_config* c) {
  return c->batch >= 1 && c->heads >= 1 && c->recent >= 0 && c->heavy >= 0 &&
         (int64_t)c->recent + c->heavy >= 1 &&
         (c->policy == H2O_POLICY_H2O || c->policy == H2O_POLICY_STATIC || c->policy == H2O_POLICY_NAIVE) &&
         (c->steps_mode == H2O_STEPS_AUTO || c->steps_mode == H2O_STEPS_PER_STEP ||
          c->steps_mode == H2O_STEPS_PERSISTENT || c->steps_mode == H2O_STEPS_RESIDENT) &&
         c->max_prompt >= 0 && c->max_prompt <= H2O_MAX_PROMPT &&
         (c->kv_dtype == H2O_F32 || c->kv_dtype == H2O_BF16) &&
         isfinite(c->scale) && c->scale >= 0.f && c->start_pos >= 0 && c->start_live >= 0 &&
         (c->decode_waves == 0 || c->decode_waves == 1 || c->decode_waves == 2 ||
          c->decode_waves == 4 || c->decode_waves == 8) &&
         c->decode_split >= 0 && c->decode_split <= 64 &&
         (c->cache_dtype == H2O_CACHE_INPUT ||
          (c->cache_dtype == H2O_CACHE_E4M3 && c->kv_dtype == H2O_BF16));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

h2o_status from_hip(hipError_t e) {
  if (e == hipSuccess) return H2O_OK;
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return H2O_ERR_OOM;
  return H2O_ERR_HIP;
}

}  // namespace

extern "C" {

h2o_status h2o_create(const h2o_config* cfg, const h2o_state* state, h2o_ctx** out) {
  if (!cfg || !state || !out) return H2O_ERR_INVALID;
  if (!state->k_slots || !state->v_slots || !state->score || !state->pos) return H2O_ERR_INVALID;
  if (!aligned16(state->k_slots) || !aligned16(state->v_slots) || !aligned16(state->score) ||
      !aligned16(state->pos))
    return H2O_ERR_INVALID;
  if (!valid_dims(cfg)) return H2O_ERR_INVALID;
  if (cfg->cache_dtype == H2O_CACHE_E4M3 &&
      (!state->k_scale || !state->v_scale || !aligned16(state->k_scale) || !aligned16(state->v_scale)))
    return H2O_ERR_INVALID;
  if (cfg->head_dim != 64 && cfg->head_dim != 96 && cfg->head_dim != 128) return H2O_ERR_UNSUPPORTED;
  const int64_t k = (int64_t)cfg->recent + cfg->heavy;
  if (k > H2O_MAX_K) return H2O_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)cfg->batch * cfg->heads;
  if (units > INT32_MAX / 8) return H2O_ERR_INVALID;   // grid size and 32-bit index headroom
  // Adopted state: the ring must hold min(t, r) rows and at most k are live.
  const int32_t t0 = cfg->start_pos, n0 = cfg->start_live;
  if (n0 == 0) {
    if (t0 != 0) return H2O_ERR_INVALID;
  } else {
    const int64_t ring = t0 < cfg->recent ? t0 : cfg->recent;
    const int64_t cap = t0 < k ? t0 : k;
    if (n0 < ring || n0 > cap) return H2O_ERR_INVALID;
    if (t0 >= INT32_MAX - 1) return H2O_ERR_STATE;
  }

  h2o_ctx* c = new (std::nothrow) h2o_ctx();
  if (!c) return H2O_ERR_OOM;
  c->cfg = *cfg;
  c->st = *state;
  c->k = (int32_t)k;
  c->waves = cfg->decode_waves ? cfg->decode_waves : h2o::decode_waves_auto((int)units);
  // the single-step kernels keep k + 1 logits in LDS beside their static arrays
  auto lds_ok = [&](int w) {
    return h2o::decode_static_lds(cfg->kv_dtype, cfg->cache_dtype, cfg->head_dim, w) + (size_t)(k + 1) * 4 <=
           h2o::kMaxLds;
  };
  while (!cfg->decode_waves && c->waves > 1 && !lds_ok(c->waves)) c->waves /= 2;
  if (!lds_ok(c->waves)) {
    delete c;
    return H2O_ERR_UNSUPPORTED;
  }
  const float scale = cfg->scale > 0.f ? cfg->scale : 1.f / sqrtf((float)cfg->head_dim);
  c->scale_log2 = scale * kLog2e;
  c->t = t0;
  c->n_live = n0;
  c->has_state = n0 > 0;
  c->stride = (int32_t)(((int64_t)cfg->max_prompt + 15) / 16 * 16);
  c->scratch = nullptr;
  c->split_mem = nullptr;
  c->multi_capacity = -1;
  c->cus = -1;
  c->lds_limit = -1;
  c->split = h2o::SplitScratch{nullptr, nullptr, nullptr, 1};
  int cus = 256;  // compute units of the current device (MI355X: 256), asked only when
                  // the automatic choice could split
  if (!cfg->decode_split && c->waves >= 8 && k >= 768) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
  }
  const int splits =
      cfg->decode_split ? cfg->decode_split : h2o::decode_split_auto((int)units, c->waves, c->k, cus);
  if (cfg->max_prompt > 0) {
    const size_t bytes = (size_t)2 * units * c->stride * sizeof(float);
    const hipError_t e = hipMalloc((void**)&c->scratch, bytes);
    if (e != hipSuccess) {
      delete c;
      return from_hip(e);
    }
  }
  if (splits > 1) {
    const size_t n_part = (size_t)units * splits * (cfg->head_dim + 2);
    const size_t n_logit = (size_t)units * (k + 1);
    const size_t bytes = (n_part + n_logit) * sizeof(float) + (size_t)units * sizeof(unsigned);
    hipError_t e = hipMalloc(&c->split_mem, bytes);
    if (e == hipSuccess) e = hipMemset(c->split_mem, 0, bytes);
    if (e != hipSuccess) {
      if (c->split_mem) (void)hipFree(c->split_mem);
      if (c->scratch) (void)hipFree(c->scratch);
      delete c;
      return from_hip(e);
    }
    c->split.partials = (float*)c->split_mem;
    c->split.logits = c->split.partials + n_part;
    c->split.counters = (unsigned*)(c->split.logits + n_logit);
    c->split.splits = splits;
  }
  *out = c;
  return H2O_OK;
}

h2o_status h2o_prefill(h2o_ctx* ctx, const void* q, const void* k, const void* v,
                       int32_t prompt_len, void* stream) {
  return h2o_prefill_with_output(ctx, q, k, v, prompt_len, nullptr, stream);
}

h2o_status h2o_prefill_with_output(h2o_ctx* ctx, const void* q, const void* k, const void* v,
                                   int32_t prompt_len, float* out, void* stream) {
  const h2o_status st = h2o::check_prefill(ctx, q, k, v, prompt_len, out);
  if (st != H2O_OK) return st;
  if (prompt_len > ctx->cfg.max_prompt) return H2O_ERR_INVALID;
  const size_t units = (size_t)ctx->cfg.batch * ctx->cfg.heads;
  return h2o::run_prefill(ctx, q, k, v, prompt_len, out, ctx->scratch, ctx->scratch + units * ctx->stride,
                          ctx->stride, stream);
}

}  // extern "C"

namespace h2o {

h2o_status check_prefill(const h2o_ctx* ctx, const void* q, const void* k, const void* v, int32_t prompt_len,
                         const float* out) {
  if (!ctx || !q || !k || !v) return H2O_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (out && !aligned16(out))) return H2O_ERR_INVALID;
  if (prompt_len < 1 || prompt_len > H2O_MAX_PROMPT) return H2O_ERR_INVALID;
  const int64_t units = (int64_t)ctx->cfg.batch * ctx->cfg.heads;
  if ((int64_t)((prompt_len + 63) / 64) * units > INT32_MAX) return H2O_ERR_INVALID;
  return H2O_OK;
}

h2o_status run_prefill(h2o_ctx* ctx, const void* q, const void* k, const void* v, int32_t prompt_len, float* out,
                       float* row_lse, float* colsum, int32_t stride, void* stream) {
  const size_t units = (size_t)ctx->cfg.batch * ctx->cfg.heads;
  PrefillArgs a;
  a.pq = q;
  a.pk = k;
  a.pv = v;
  a.k_slots = ctx->st.k_slots;
  a.v_slots = ctx->st.v_slots;
  a.score = ctx->st.score;
  a.pos = ctx->st.pos;
  a.k_scale = ctx->st.k_scale;
  a.v_scale = ctx->st.v_scale;
  a.row_lse = row_lse;
  a.colsum = colsum;
  a.out = out;
  a.units = (int32_t)units;
  a.stride = stride;
  a.P = prompt_len;
  a.k = ctx->k;
  a.r = ctx->cfg.recent;
  a.h = ctx->cfg.heavy;
  a.scale_log2 = ctx->scale_log2;
  a.last_row_only = ctx->cfg.policy == H2O_POLICY_NAIVE;
  const hipError_t e = launch_prefill(a, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype, ctx->cfg.head_dim,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return from_hip(e);
  ctx->t = prompt_len;
  ctx->n_live = prompt_len < ctx->k ? prompt_len : ctx->k;
  ctx->has_state = true;
  return H2O_OK;
}

}  // namespace h2o

namespace {

// Kernel arguments of the step at the ctx's current position.
h2o::DecodeArgs step_args(const h2o_ctx* ctx, const void* q, const void* k_new, const void* v_new, float* out,
                          int32_t* evicted_pos) {
  const int32_t r = ctx->cfg.recent;
  const int32_t n_ring = ctx->t < r ? ctx->t : r;
  h2o::DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_slots = ctx->st.k_slots;
  a.v_slots = ctx->st.v_slots;
  a.score = ctx->st.score;
  a.pos = ctx->st.pos;
  a.k_scale = ctx->st.k_scale;
  a.v_scale = ctx->st.v_scale;
  a.out = out;
  a.evicted = evicted_pos;
  a.units = ctx->cfg.batch * ctx->cfg.heads;
  a.k = ctx->k;
  a.r = r;
  a.t = ctx->t;
  a.n_ring = n_ring;
  a.n_heavy = ctx->n_live - n_ring;
  a.scale_log2 = ctx->scale_log2;
  a.policy = ctx->cfg.policy;
  return a;
}

// Enqueue one decode step at the ctx's current position and advance it.
h2o_status enqueue_step(h2o_ctx* ctx, const void* q, const void* k_new, const void* v_new,
                        float* out, int32_t* evicted_pos, hipStream_t stream) {
  const h2o::DecodeArgs a = step_args(ctx, q, k_new, v_new, out, evicted_pos);
  const hipError_t e = h2o::launch_decode(a, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype,
                                          ctx->cfg.head_dim, ctx->waves, &ctx->split, stream);
  if (e != hipSuccess) return from_hip(e);
  ctx->t += 1;
  if (ctx->n_live < ctx->k) ctx->n_live += 1;
  return H2O_OK;
}

bool step_args_ok(const void* q, const void* k_new, const void* v_new, const float* out,
                  const int32_t* evicted_pos) {
  return q && k_new && v_new && out && aligned16(q) && aligned16(k_new) && aligned16(v_new) &&
         aligned16(out) && ((uintptr_t)evicted_pos & 3u) == 0;
}

}  // namespace

extern "C" {

h2o_status h2o_decode_step(h2o_ctx* ctx, const void* q, const void* k_new, const void* v_new,
                           float* out, int32_t* evicted_pos, void* stream) {
  if (!ctx || !step_args_ok(q, k_new, v_new, out, evicted_pos)) return H2O_ERR_INVALID;
  if (!ctx->has_state) return H2O_ERR_STATE;
  if (ctx->t >= INT32_MAX - 1) return H2O_ERR_STATE;
  return enqueue_step(ctx, q, k_new, v_new, out, evicted_pos, (hipStream_t)stream);
}

namespace {

// Compute units and per-workgroup LDS of the ctx's device, asked once.
void query_device(h2o_ctx* ctx) {
  if (ctx->cus >= 0) return;
  int dev = 0, cus = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) lds = 0;
  ctx->cus = cus > 0 ? cus : 0;
  ctx->lds_limit = lds > 0 ? lds : 0;
}

// The resident multi-step kernel applies: every unit's workgroup, holding all
// of the unit's rows in LDS, gets a compute unit of its own.
bool resident_fits(h2o_ctx* ctx) {
  if (ctx->split.splits >= 2) return false;
  query_device(ctx);
  const int64_t units = (int64_t)ctx->cfg.batch * ctx->cfg.heads;
  return units <= ctx->cus &&
         (int64_t)h2o::decode_resident_lds(ctx->k, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype, ctx->cfg.head_dim,
                                           ctx->waves) <= ctx->lds_limit &&
         h2o::decode_multi_fits(ctx->k, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype, ctx->cfg.head_dim, ctx->waves);
}

// How h2o_decode_steps runs n_steps: H2O_STEPS_RESIDENT, H2O_STEPS_PERSISTENT
// (one launch) or H2O_STEPS_PER_STEP.
int steps_plan(h2o_ctx* ctx, int32_t n_steps) {
  const int mode = ctx->cfg.steps_mode;
  if (n_steps < 2 || ctx->split.splits >= 2 || mode == H2O_STEPS_PER_STEP) return H2O_STEPS_PER_STEP;
  if ((mode == H2O_STEPS_AUTO || mode == H2O_STEPS_RESIDENT) && resident_fits(ctx)) return H2O_STEPS_RESIDENT;
  if (mode == H2O_STEPS_RESIDENT) return H2O_STEPS_PER_STEP;
  if (!h2o::decode_multi_fits(ctx->k, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype, ctx->cfg.head_dim, ctx->waves))
    return H2O_STEPS_PER_STEP;
  if (mode == H2O_STEPS_PERSISTENT) return H2O_STEPS_PERSISTENT;
  // Automatic: one launch when every unit's workgroup is resident at once
  // (else a unit waits for whole launches of the others), and either the
  // decode has several wavefronts per unit or a step moves little data.
  // Measured on MI355X: ahead of per-step launches at 2, 4 and 8 wavefronts
  // per unit on every workload tried, behind with single-wave units of a
  // bf16 cache (3584 units, k = 410: 127 against 117 us per step).
  const size_t row_bytes = (size_t)ctx->cfg.head_dim *
                           (ctx->cfg.cache_dtype == H2O_CACHE_E4M3 ? 1 : ctx->cfg.kv_dtype == H2O_BF16 ? 2 : 4);
  const size_t n_units = (size_t)ctx->cfg.batch * ctx->cfg.heads;
  const size_t step_bytes = n_units * ctx->k * 2 * row_bytes;  // cached K/V bytes one step streams
  if (ctx->waves == 1 && step_bytes > ((size_t)64 << 20)) return H2O_STEPS_PER_STEP;
  if (ctx->multi_capacity < 0) {
    query_device(ctx);
    const int per_cu = h2o::decode_multi_per_cu(ctx->k, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype,
                                                ctx->cfg.head_dim, ctx->waves);
    ctx->multi_capacity = per_cu > 0 ? (int64_t)per_cu * ctx->cus : 0;
  }
  return (int64_t)n_units <= ctx->multi_capacity ? H2O_STEPS_PERSISTENT : H2O_STEPS_PER_STEP;
}

}  // namespace

h2o_status h2o_decode_steps(h2o_ctx* ctx, int32_t n_steps, const void* q, const void* k_new,
                            const void* v_new, float* out, int32_t* evicted_pos, void* stream) {
  if (!ctx || n_steps < 1 || !step_args_ok(q, k_new, v_new, out, evicted_pos)) return H2O_ERR_INVALID;
  if (!ctx->has_state) return H2O_ERR_STATE;
  if ((int64_t)ctx->t + n_steps >= INT32_MAX - 1) return H2O_ERR_STATE;
  const int plan = steps_plan(ctx, n_steps);
  if (plan != H2O_STEPS_PER_STEP) {
    // one launch carries every unit through all n_steps (resident: with its rows in LDS)
    const h2o::DecodeArgs a = step_args(ctx, q, k_new, v_new, out, evicted_pos);
    const hipError_t e =
        h2o::launch_decode_multi(a, ctx->cfg.kv_dtype, ctx->cfg.cache_dtype, ctx->cfg.head_dim, ctx->waves,
                                 n_steps, ctx->n_live, plan == H2O_STEPS_RESIDENT, (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e);
    ctx->t += n_steps;
    ctx->n_live = (int64_t)ctx->n_live + n_steps < ctx->k ? ctx->n_live + n_steps : ctx->k;
    return H2O_OK;
  }
  const size_t n_units = (size_t)ctx->cfg.batch * ctx->cfg.heads;
  const size_t in_step = n_units * ctx->cfg.head_dim * (ctx->cfg.kv_dtype == H2O_BF16 ? 2 : 4);
  const size_t out_step = n_units * ctx->cfg.head_dim;
  for (int32_t s = 0; s < n_steps; ++s) {
    const h2o_status st = enqueue_step(
        ctx, (const char*)q + s * in_step, (const char*)k_new + s * in_step,
        (const char*)v_new + s * in_step, out + s * out_step,
        evicted_pos ? evicted_pos + s * n_units : nullptr, (hipStream_t)stream);
    if (st != H2O_OK) return st;
  }
  return H2O_OK;
}

h2o_status h2o_steps_launch(h2o_ctx* ctx, int32_t n_steps, int32_t* mode) {
  if (!ctx || n_steps < 1 || !mode) return H2O_ERR_INVALID;
  *mode = steps_plan(ctx, n_steps);
  return H2O_OK;
}

h2o_status h2o_query(const h2o_ctx* ctx, int32_t* next_pos, int32_t* n_live) {
  if (!ctx) return H2O_ERR_INVALID;
  if (next_pos) *next_pos = ctx->t;
  if (n_live) *n_live = ctx->n_live;
  return H2O_OK;
}

h2o_status h2o_launch_shape(const h2o_ctx* ctx, int32_t* decode_waves, int32_t* decode_split) {
  if (!ctx) return H2O_ERR_INVALID;
  if (decode_waves) *decode_waves = ctx->waves;
  if (decode_split) *decode_split = ctx->split.splits;
  return H2O_OK;
}

h2o_status h2o_destroy(h2o_ctx* ctx) {
  if (!ctx) return H2O_OK;
  hipError_t e = hipSuccess;
  if (ctx->scratch) e = hipFree(ctx->scratch);
  if (ctx->split_mem) {
    const hipError_t e2 = hipFree(ctx->split_mem);
    if (e == hipSuccess) e = e2;
  }
  delete ctx;
  return from_hip(e);
}

const char* h2o_status_string(h2o_status status) {
  switch (status) {
    case H2O_OK: return "ok";
    case H2O_ERR_INVALID: return "invalid argument";
    case H2O_ERR_UNSUPPORTED: return "unsupported configuration";
    case H2O_ERR_STATE: return "invalid call order or position overflow";
    case H2O_ERR_OOM: return "out of device memory";
    case H2O_ERR_HIP: return "HIP runtime error";
    case H2O_ERR_TOO_LARGE: return "needs more scratch than the fixed no-allocation buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
