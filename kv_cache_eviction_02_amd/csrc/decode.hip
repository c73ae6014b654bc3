// Fused H2O decode step for gfx950: attention over the cached slots and the new
// token, accumulated-score update, eviction argmin and in-place admission.
//
// Method (H2O summary "H2O: Heavy-Hitter Oracle for Efficient Generative
// Inference", "Algorithm / figure walkthrough" steps 2-4 and "The mechanism",
// H2O eviction with Definition 4.3):
//   l_j = scale * q . K_j over the live slots and the new token (self);
//   p = softmax(l); out = sum_j p_j V_j;
//   score_j += p_j; the new token's score is p_self;
//   when the cache was full (k live slots), evict the slot with the smallest
//   (score, position) among the heavy slots and the ring slot whose position
//   t - r just left the protected window.
//
// Two kernels share the streaming loop and the final score/eviction code:
//
// decode_kernel: one workgroup per (batch, head) unit.  K and V rows are
//   streamed once with 16-byte non-temporal loads, a row spread over
//   D*sizeof(T)/16 consecutive lanes (16 lanes for bf16 d = 128, 12 of a
//   16-lane group for d = 96, 8 for d = 64).  Each row group keeps an online
//   softmax (running max, running sum, running output), so K and V are read in
//   the same pass; the groups are merged through LDS at the end.  Logits (log2
//   domain) stay in LDS for the exact score update.  The argmin is a
//   deterministic u64 minimum over (score bits << 32 | position): non-negative
//   float bit patterns order like unsigned integers, so equal scores send the
//   older position out.  The ring row that may move to the victim's slot and
//   the new token's row are kept in LDS from the streaming pass, so admission
//   writes at most two rows without reading them again.
//
// decode_split_kernel: for batches with few units, S workgroups share a unit,
//   each streaming a contiguous range of its rows.  Every workgroup writes its
//   partial (max, sum, output) and its logits to scratch and increments the
//   unit's arrival counter; the last to arrive combines the partials, runs the
//   score update and eviction, and resets the counter.  No workgroup waits for
//   another.
#include <float.h>
#include <math.h>

#include "common.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int ceil_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

__device__ inline unsigned long long shfl_xor_u64(unsigned long long x, int mask) {
  const uint32_t lo = __shfl_xor((uint32_t)x, mask, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), mask, 64);
  return ((unsigned long long)hi << 32) | lo;
}

template <typename T, int D, int NW>
struct Geo {
  using E = Elem<T>;
  static constexpr int EPL = E::kPer16B;     // elements per lane per row
  static constexpr int LPR = D / EPL;        // lanes holding one row
  static constexpr int G = ceil_pow2(LPR);   // lanes per row group
  static constexpr int RW = 64 / G;          // rows per wave per batch
  static constexpr int NG = NW * RW;         // row groups per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = D * E::kBytes;
  static constexpr int PF = 8;               // slots per thread prefetched for the score update
  static_assert(LPR * EPL == D && G <= 64, "row mapping");
};

// One unit's step as seen by every thread.
struct StepView {
  int k, r, t, n_ring, n_heavy, n_live, n_att, ring_slot;
  bool full, ring_live;
  __device__ StepView(const DecodeArgs& a)
      : k(a.k), r(a.r), t(a.t), n_ring(a.n_ring), n_heavy(a.n_heavy),
        n_live(a.n_ring + a.n_heavy), n_att(a.n_ring + a.n_heavy + 1), ring_slot(a.t % a.r),
        full(a.n_ring + a.n_heavy == a.k), ring_live(a.t % a.r < a.n_ring) {}
  // Logical row j: live ring slots [0, n_ring), then live heavy slots; row n_live is the new token.
  __device__ int slot_of(int j) const { return j < n_ring ? j : r + (j - n_ring); }
  __device__ bool is_cand(int s) const { return full && (s >= r || s == ring_slot); }
};

// Per-unit pointers.
template <int ROWB>
struct UnitPtrs {
  char* K;
  char* V;
  const char* kn;
  const char* vn;
  const char* q;
  float* score;
  int32_t* pos;
  __device__ UnitPtrs(const DecodeArgs& a, int unit, int k) {
    const size_t ubase = (size_t)unit * k;
    K = (char*)a.k_slots + ubase * ROWB;
    V = (char*)a.v_slots + ubase * ROWB;
    kn = (const char*)a.k_new + (size_t)unit * ROWB;
    vn = (const char*)a.v_new + (size_t)unit * ROWB;
    q = (const char*)a.q + (size_t)unit * ROWB;
    score = a.score + ubase;
    pos = a.pos + ubase;
  }
};

// Streams logical rows [lo, hi): logit of each row into s_logit[j] (log2
// domain), per-row-group online softmax into (m, lsum, o).  The new token's row
// and the ring row leaving the window are copied into the LDS stash when they
// fall in the range.  Loads are unconditional (rows outside the range and idle
// lanes re-read a valid row and are masked out) so the compiler tracks
// outstanding loads exactly; the next row batch is in flight while the current
// one is consumed.
template <typename T, int D, int NW>
__device__ __forceinline__ void stream_rows(const StepView& v, const UnitPtrs<Geo<T, D, NW>::ROWB>& u,
                                            int lo, int hi, const float* qf, float scale_log2,
                                            float* s_logit, uint4 (*s_ring)[Geo<T, D, NW>::LPR],
                                            uint4 (*s_self)[Geo<T, D, NW>::LPR], float& m,
                                            float& lsum, float* o) {
  using GG = Geo<T, D, NW>;
  using E = typename GG::E;
  constexpr int EPL = GG::EPL, G = GG::G, RW = GG::RW, NG = GG::NG, LPR = GG::LPR;
  const int lane = threadIdx.x & 63;
  const int gl = lane & (G - 1);
  const int grp = (threadIdx.x >> 6) * RW + lane / G;
  const bool act = gl < LPR;
  const int chunk = act ? gl : 0;

  auto fetch = [&](int base, uint4& kr, uint4& vr) {
    const int j = base + grp;
    const char* kp = u.kn;
    const char* vp = u.vn;
    if (j < v.n_live && j < hi) {
      const size_t off = (size_t)v.slot_of(j) * GG::ROWB;
      kp = u.K + off;
      vp = u.V + off;
    }
    kr = load16_stream(kp + chunk * 16);
    vr = load16_stream(vp + chunk * 16);
  };
  auto consume = [&](int base, const uint4& kr, const uint4& vr) {
    float kf[EPL];
    E::unpack(kr, kf);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) d = fmaf(qf[e], kf[e], d);  // qf is 0 on idle lanes
    d = group_sum<G>(d);
    const int j = base + grp;
    const bool valid = j < hi;
    const float lg = valid ? d * scale_log2 : -INFINITY;
    if (valid) {
      if (gl == 0) s_logit[j] = lg;
      if (act) {
        if (j == v.n_live) {
          s_self[0][gl] = kr;
          s_self[1][gl] = vr;
        } else if (v.ring_live && j == v.ring_slot) {
          s_ring[0][gl] = kr;
          s_ring[1][gl] = vr;
        }
      }
    }
    const float mn = fmaxf(m, lg);
    if (mn > -INFINITY) {
      const float alpha = fast_exp2(m - mn);
      const float p = fast_exp2(lg - mn);  // 0 for rows outside the range
      float vf[EPL];
      E::unpack(vr, vf);
      lsum = fmaf(lsum, alpha, p);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e] * alpha);
      m = mn;
    }
  };

  uint4 ka, va, kb, vb;
  fetch(lo, ka, va);
  for (int base = lo; base < hi; base += 2 * NG) {
    fetch(base + NG, kb, vb);
    consume(base, ka, va);
    fetch(base + 2 * NG, ka, va);
    consume(base + NG, kb, vb);
  }
}

// Workgroup merge of the row groups: leaves M (block max), the group weights
// and L (block sum) in registers of every thread; s_o keeps the group outputs.
template <int NG, int D>
struct GroupMerge {
  float M, L;
  float wg[NG];
};

template <typename T, int D, int NW>
__device__ __forceinline__ GroupMerge<Geo<T, D, NW>::NG, D> merge_groups(
    float m, float lsum, const float* o, float (*s_o)[D], float* s_m, float* s_l) {
  using GG = Geo<T, D, NW>;
  constexpr int EPL = GG::EPL, G = GG::G, RW = GG::RW, NG = GG::NG, LPR = GG::LPR;
  const int lane = threadIdx.x & 63;
  const int gl = lane & (G - 1);
  const int grp = (threadIdx.x >> 6) * RW + lane / G;
  if (gl == 0) {
    s_m[grp] = m;
    s_l[grp] = lsum;
  }
  if (gl < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_o[grp][gl * EPL + e] = o[e];
  }
  __syncthreads();
  GroupMerge<NG, D> r;
  r.M = -INFINITY;
#pragma unroll
  for (int g = 0; g < NG; ++g) r.M = fmaxf(r.M, s_m[g]);
  r.L = 0.f;
  const float base = r.M == -INFINITY ? 0.f : r.M;  // an empty range: every weight 0
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    r.wg[g] = fast_exp2(s_m[g] - base);
    r.L = fmaf(s_l[g], r.wg[g], r.L);
  }
  return r;
}

// Score update, eviction argmin and admission for one unit, given the exact
// softmax max M and 1/L.  Logits of rows [0, n_att) are in s_logit; the
// scores this thread owns were prefetched into sc_pf / ps_pf; the ring row and
// the new token's row are in the LDS stash.
template <typename T, int D, int NW>
__device__ __forceinline__ void finish_step(const StepView& v, const UnitPtrs<Geo<T, D, NW>::ROWB>& u,
                                            float M, float invL, float* s_logit, const float* sc_pf,
                                            const int* ps_pf, uint4 (*s_ring)[Geo<T, D, NW>::LPR],
                                            uint4 (*s_self)[Geo<T, D, NW>::LPR],
                                            unsigned long long* s_key, int* s_victim,
                                            int32_t* evicted, int unit) {
  using GG = Geo<T, D, NW>;
  constexpr int NT = GG::NT, PF = GG::PF, LPR = GG::LPR, ROWB = GG::ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float p_self = fast_exp2(s_logit[v.n_live] - M) * invL;

  unsigned long long best = ~0ull;
  int best_slot = -1;
  auto update = [&](int j, float old, int ps) {
    const int s = v.slot_of(j);
    const float ns = old + fast_exp2(s_logit[j] - M) * invL;
    s_logit[j] = ns;
    if (v.is_cand(s)) {
      const unsigned long long key = ((unsigned long long)__float_as_uint(ns) << 32) | (uint32_t)ps;
      if (key < best) {
        best = key;
        best_slot = s;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int j = tid + i * NT;
    if (j < v.n_live) update(j, sc_pf[i], ps_pf[i]);
  }
  for (int j = tid + PF * NT; j < v.n_live; j += NT) {
    const int s = v.slot_of(j);
    update(j, u.score[s], v.is_cand(s) ? u.pos[s] : 0);
  }

  unsigned long long vkey = ~0ull;
  if (v.full) {
    unsigned long long w = best;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const unsigned long long other = shfl_xor_u64(w, off);
      w = other < w ? other : w;
    }
    if (lane == 0) s_key[wave] = w;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) vkey = s_key[i] < vkey ? s_key[i] : vkey;
    if (best_slot >= 0 && best == vkey) *s_victim = best_slot;
  }
  __syncthreads();

  // Where the row leaving the window goes: the victim's heavy slot, or the next
  // free heavy slot while the cache is not yet full; -1 if it is dropped or
  // still inside the window.
  int dst = -1;
  if (v.full) {
    if (*s_victim != v.ring_slot) dst = *s_victim;
  } else if (v.ring_live) {
    dst = v.r + v.n_heavy;
  }

  auto write_score = [&](int j) {
    const int s = v.slot_of(j);
    if (s != v.ring_slot && s != dst) u.score[s] = s_logit[j];
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int j = tid + i * NT;
    if (j < v.n_live) write_score(j);
  }
  for (int j = tid + PF * NT; j < v.n_live; j += NT) write_score(j);

  if (tid == 0) {
    if (dst >= 0) {
      u.score[dst] = s_logit[v.ring_slot];
      u.pos[dst] = v.t - v.r;
    }
    u.score[v.ring_slot] = p_self;
    u.pos[v.ring_slot] = v.t;
    if (evicted) evicted[unit] = v.full ? (int32_t)(uint32_t)vkey : -1;
  }
  if (tid < LPR) {
    if (dst >= 0) {
      store16(u.K + (size_t)dst * ROWB + tid * 16, s_ring[0][tid]);
      store16(u.V + (size_t)dst * ROWB + tid * 16, s_ring[1][tid]);
    }
    store16(u.K + (size_t)v.ring_slot * ROWB + tid * 16, s_self[0][tid]);
    store16(u.V + (size_t)v.ring_slot * ROWB + tid * 16, s_self[1][tid]);
  }
}

// Prefetch of the scores a thread will update, and of the candidates' positions.
template <typename T, int D, int NW>
__device__ __forceinline__ void prefetch_scores(const StepView& v, const UnitPtrs<Geo<T, D, NW>::ROWB>& u,
                                                float* sc_pf, int* ps_pf) {
  using GG = Geo<T, D, NW>;
#pragma unroll
  for (int i = 0; i < GG::PF; ++i) {
    const int j = threadIdx.x + i * GG::NT;
    sc_pf[i] = 0.f;
    ps_pf[i] = 0;
    if (j < v.n_live) {
      const int s = v.slot_of(j);
      sc_pf[i] = u.score[s];
      if (v.is_cand(s)) ps_pf[i] = u.pos[s];
    }
  }
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using GG = Geo<T, D, NW>;
  using E = typename GG::E;
  constexpr int EPL = GG::EPL, LPR = GG::LPR, NG = GG::NG, NT = GG::NT, PF = GG::PF;

  __shared__ float s_o[NG][D];
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];
  __shared__ uint4 s_ring[2][LPR];  // K, V of the ring slot leaving the window
  __shared__ uint4 s_self[2][LPR];  // K, V of the decoded token
  __shared__ unsigned long long s_key[NW];
  __shared__ int s_victim;
  extern __shared__ float s_logit[];  // [n_live + 1] logits, later updated scores

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const StepView v(a);
  const UnitPtrs<GG::ROWB> u(a, unit, v.k);
  const int gl = (tid & 63) & (GG::G - 1);
  const bool act = gl < LPR;

  if (tid == 0) s_victim = v.ring_slot;  // overwritten by the argmin owner when the cache is full

  float qf[EPL];
  E::unpack(act ? load16(u.q + gl * 16) : make_uint4(0, 0, 0, 0), qf);
  float sc_pf[PF];
  int ps_pf[PF];
  prefetch_scores<T, D, NW>(v, u, sc_pf, ps_pf);

  float m = -INFINITY, lsum = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  stream_rows<T, D, NW>(v, u, 0, v.n_att, qf, a.scale_log2, s_logit, s_ring, s_self, m, lsum, o);

  const GroupMerge<NG, D> gm = merge_groups<T, D, NW>(m, lsum, o, s_o, s_m, s_l);
  const float invL = 1.f / gm.L;
  for (int c = tid; c < D; c += NT) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc = fmaf(s_o[g][c], gm.wg[g], acc);
    a.out[(size_t)unit * D + c] = acc * invL;
  }
  finish_step<T, D, NW>(v, u, gm.M, invL, s_logit, sc_pf, ps_pf, s_ring, s_self, s_key, &s_victim,
                        a.evicted, unit);
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(DecodeArgs a, SplitScratch sp) {
  using GG = Geo<T, D, NW>;
  using E = typename GG::E;
  constexpr int EPL = GG::EPL, LPR = GG::LPR, NG = GG::NG, NT = GG::NT, PF = GG::PF;
  constexpr int ROWB = GG::ROWB;

  __shared__ float s_o[NG][D];
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];
  __shared__ uint4 s_ring[2][LPR];
  __shared__ uint4 s_self[2][LPR];
  __shared__ unsigned long long s_key[NW];
  __shared__ int s_victim;
  __shared__ int s_last;
  extern __shared__ float s_logit[];  // [n_live + 1]

  const int S = sp.splits;
  const int unit = blockIdx.x / S;
  const int part = blockIdx.x % S;
  const int tid = threadIdx.x;
  const StepView v(a);
  const UnitPtrs<ROWB> u(a, unit, v.k);
  const int gl = (tid & 63) & (GG::G - 1);
  const bool act = gl < LPR;

  if (tid == 0) s_victim = v.ring_slot;

  float qf[EPL];
  E::unpack(act ? load16(u.q + gl * 16) : make_uint4(0, 0, 0, 0), qf);
  float sc_pf[PF];
  int ps_pf[PF];
  prefetch_scores<T, D, NW>(v, u, sc_pf, ps_pf);

  const int per = (v.n_att + S - 1) / S;
  const int lo = min(v.n_att, part * per);
  const int hi = min(v.n_att, lo + per);
  float m = -INFINITY, lsum = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  stream_rows<T, D, NW>(v, u, lo, hi, qf, a.scale_log2, s_logit, s_ring, s_self, m, lsum, o);
  const GroupMerge<NG, D> gm = merge_groups<T, D, NW>(m, lsum, o, s_o, s_m, s_l);

  // This workgroup's partial: max, sum, output relative to its max; its logits.
  float* pp = sp.partials + ((size_t)unit * S + part) * (D + 2);
  if (tid == 0) {
    pp[0] = gm.M;
    pp[1] = gm.L;
  }
  for (int c = tid; c < D; c += NT) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc = fmaf(s_o[g][c], gm.wg[g], acc);
    pp[2 + c] = acc;
  }
  float* lg = sp.logits + (size_t)unit * (v.k + 1);
  for (int j = lo + tid; j < hi; j += NT) lg[j] = s_logit[j];

  // Publish, count arrivals; the last workgroup of the unit finishes the step.
  // The workgroup barrier completes every thread's stores; one agent-scope
  // release by thread 0 then makes them visible to the other XCDs before the
  // arrival is counted (a device-scope fence writes back the XCD's L2, so it
  // is issued once per workgroup, not once per thread).
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned prev = __hip_atomic_fetch_add(sp.counters + unit, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(S - 1);
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_last) return;

  // Combine the partials.
  const float* up = sp.partials + (size_t)unit * S * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < S; ++c) M = fmaxf(M, up[(size_t)c * (D + 2)]);
  float L = 0.f;
  for (int c = 0; c < S; ++c) {
    const float* q = up + (size_t)c * (D + 2);
    L = fmaf(q[1], fast_exp2(q[0] - M), L);
  }
  const float invL = 1.f / L;
  for (int d = tid; d < D; d += NT) {
    float acc = 0.f;
    for (int c = 0; c < S; ++c) {
      const float* q = up + (size_t)c * (D + 2);
      acc = fmaf(q[2 + d], fast_exp2(q[0] - M), acc);
    }
    a.out[(size_t)unit * D + d] = acc * invL;
  }
  // All logits, and the two rows the admission writes (still intact: only this
  // workgroup writes the unit's state).
  for (int j = tid; j < v.n_att; j += NT) s_logit[j] = lg[j];
  if (tid < LPR) {
    s_self[0][tid] = load16(u.kn + tid * 16);
    s_self[1][tid] = load16(u.vn + tid * 16);
    if (v.ring_live) {
      s_ring[0][tid] = load16(u.K + (size_t)v.ring_slot * ROWB + tid * 16);
      s_ring[1][tid] = load16(u.V + (size_t)v.ring_slot * ROWB + tid * 16);
    }
  }
  __syncthreads();
  finish_step<T, D, NW>(v, u, M, invL, s_logit, sc_pf, ps_pf, s_ring, s_self, s_key, &s_victim,
                        a.evicted, unit);
  if (tid == 0) sp.counters[unit] = 0u;  // ready for the next step
}

template <typename T, int D, int NW>
hipError_t launch_nw(const DecodeArgs& a, const SplitScratch* sp, hipStream_t s) {
  const int n_live = a.n_ring + a.n_heavy;
  const size_t lds = (size_t)(n_live + 1) * sizeof(float);
  if (sp && sp->splits > 1) {
    hipLaunchKernelGGL((decode_split_kernel<T, D, NW>), dim3(a.units * sp->splits), dim3(NW * 64),
                       lds, s, a, *sp);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, NW>), dim3(a.units), dim3(NW * 64), lds, s, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, int waves, const SplitScratch* sp, hipStream_t s) {
  switch (waves) {
    case 1: return launch_nw<T, D, 1>(a, sp, s);
    case 2: return launch_nw<T, D, 2>(a, sp, s);
    case 4: return launch_nw<T, D, 4>(a, sp, s);
    case 8: return launch_nw<T, D, 8>(a, sp, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, int head_dim, int waves, const SplitScratch* sp,
                    hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<T, 64>(a, waves, sp, s);
    case 96: return launch_d<T, 96>(a, waves, sp, s);
    case 128: return launch_d<T, 128>(a, waves, sp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_waves_auto(int units) {
  // Aim at about four resident wavefronts per SIMD (256 CUs x 4 SIMDs).
  int w = 1;
  while (w < 8 && (long)units * w * 2 <= 4096) w *= 2;
  return w;
}

int decode_split_auto(int units, int waves) {
  (void)waves;
  (void)units;
  return 1;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int waves,
                         const SplitScratch* sp, hipStream_t s) {
  if (dtype == 0) return launch_t<float>(a, head_dim, waves, sp, s);
  if (dtype == 1) return launch_t<bf16>(a, head_dim, waves, sp, s);
  return hipErrorInvalidValue;
}

}  // namespace h2o
