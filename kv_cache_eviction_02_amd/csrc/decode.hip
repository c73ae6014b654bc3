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
// Ablations of the same step (summary, "Prior limits" and "Limitations"): the
// static policy always evicts the position leaving the window, the naive one
// replaces each score by the current weight instead of adding it, and r = 0
// (heavy-only) makes the decoded token itself a candidate.
//
// Four kernels share the streaming loop and the final score/eviction code:
//
// decode_kernel: one workgroup per (batch, head) unit.  K and V rows are
//   streamed once with 16-byte non-temporal loads, a row spread over
//   D*sizeof(C)/16 consecutive lanes (16 lanes for bf16 d = 128, 12 of a
//   16-lane group for d = 96, 8 for d = 64; E4M3 rows take half as many).  Each
//   row group keeps an online softmax (running max, running sum, running
//   output), so K and V are read in the same pass; the groups are merged
//   through LDS at the end.  Logits (log2 domain) stay in LDS for the exact
//   score update.  The argmin is a deterministic u64 minimum over (score bits
//   << 32 | position): non-negative float bit patterns order like unsigned
//   integers, so equal scores send the older position out.  The ring row that
//   may move to the victim's slot and the new token's row are kept in LDS from
//   the streaming pass, so admission writes at most two rows.
//
// decode_split_kernel: for batches with few units and long contexts, S
//   workgroups share a unit, each streaming a contiguous range of its rows.
//   Every workgroup writes its partial (max, sum, output) and its logits to
//   scratch with device-scope stores and increments the unit's arrival counter;
//   the last to arrive reads them back with device-scope loads, combines the
//   partials, runs the score update and eviction, and resets the counter.  No
//   workgroup waits for another and no cache is written back.
//
// decode_multi_kernel: n steps over tokens known in advance in one launch; each
//   workgroup carries its unit from step to step with the scores and positions
//   in LDS, so one unit's end-of-step work overlaps the others' streaming.
//
// decode_resident_kernel: the same with the unit's K and V rows held in LDS
//   for the whole launch (a long stream at small batch): a step reads only its
//   inputs from memory, and the admission writes both copies.
//
// At large batch (up to four wavefronts per unit) the admitted rows are stored
// with the non-temporal hint.
//
// E4M3 cache (C = e4m3, bf16 inputs): slots hold E4M3 codes with one float32
// scale per row; the K scale multiplies the row's logit and the V scale its
// weight.  The decoded token attends with its exact bf16 row; its codes,
// x * (448 / amax), and scale, amax / 448, are computed while the stream's
// first rows are in flight and stored on admission.
#include <float.h>
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int ceil_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Minimum of the lane's key and lane l ^ 16's (k32: l ^ 32's), in every lane.
template <bool k32>
__device__ inline unsigned long long min_pair_u64(unsigned long long x) {
  const LanePair lo = k32 ? pair32((uint32_t)x) : pair16((uint32_t)x);
  const LanePair hi = k32 ? pair32((uint32_t)(x >> 32)) : pair16((uint32_t)(x >> 32));
  const unsigned long long a = ((unsigned long long)hi.a << 32) | lo.a;
  const unsigned long long b = ((unsigned long long)hi.b << 32) | lo.b;
  return a < b ? a : b;
}

template <int CTRL>
__device__ inline unsigned long long dpp_u64(unsigned long long x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Minimum over the 64 lanes, in every lane: DPP within each row of 16 lanes
// (quad swaps, then the half-row and row mirrors), then the two cross-row
// permlane swaps.
__device__ inline unsigned long long wave_min_u64(unsigned long long w) {
  unsigned long long o;
  o = dpp_u64<kDppQuadXor1>(w);
  w = o < w ? o : w;
  o = dpp_u64<kDppQuadXor2>(w);
  w = o < w ? o : w;
  o = dpp_u64<kDppHalfMirror>(w);
  w = o < w ? o : w;
  o = dpp_u64<kDppRowMirror>(w);
  w = o < w ? o : w;
  w = min_pair_u64<false>(w);
  return min_pair_u64<true>(w);
}

// T: input element type (q, k_new, v_new); C: cache element type.
template <typename T, typename C, int D, int NW>
struct Geo {
  using EC = Elem<C>;
  using EI = Elem<T>;
  static constexpr bool kQuant = std::is_same<C, e4m3>::value;
  static constexpr int EPL = EC::kPer16B;    // elements per lane per row
  static constexpr int LPR = D / EPL;        // lanes holding one row
  static constexpr int G = ceil_pow2(LPR);   // lanes per row group
  static constexpr int RW = 64 / G;          // rows per wave per batch
  static constexpr int NG = NW * RW;         // row groups per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = D * EC::kBytes;   // cache row bytes
  static constexpr int IROWB = D * EI::kBytes;  // input row bytes
  static constexpr int ICH = EPL * EI::kBytes / 16;  // 16-byte input chunks per lane
  static constexpr int PF = 8;               // slots per thread prefetched for the score update
  // Admitted rows stored with the non-temporal hint at large batch (up to four
  // wavefronts per unit), where the caches stream far more than they hold; the
  // small batches' working sets stay in the caches, which the hint bypasses.
  static constexpr bool kNtRows = NW <= 4;
  static_assert(LPR * EPL == D && G <= 64, "row mapping");
  static_assert(!kQuant || std::is_same<T, bf16>::value, "E4M3 cache takes bf16 inputs");
};

constexpr float kLazyMax = 8.f;  // log2 units a row group's running maximum may lag
// Running maximum of a row group before its first row: finite, so that the
// weight exp2(lg - m) of a row outside the range (lg = -inf) is 0 without a
// test, and the first row raises the maximum (its rescale factor exp2(kNoMax -
// lg) is 0, as it would be from -inf).
constexpr float kNoMax = -FLT_MAX;
constexpr int kSelfVictim = -2;  // victim marker: the decoded token itself (r = 0)

// One unit's step as seen by every thread.  With r = 0 there is no ring:
// ring_slot is -1 and every slot is a heavy slot.
struct StepView {
  int k, r, t, n_ring, n_heavy, n_live, n_att, ring_slot, policy;
  bool full, ring_live;
  __device__ StepView(const DecodeArgs& a)
      : k(a.k), r(a.r), t(a.t), n_ring(a.n_ring), n_heavy(a.n_heavy),
        n_live(a.n_ring + a.n_heavy), n_att(a.n_ring + a.n_heavy + 1),
        ring_slot(a.r > 0 ? a.t % a.r : -1), policy(a.policy), full(a.n_ring + a.n_heavy == a.k),
        ring_live(a.r > 0 && a.t % a.r < a.n_ring) {}
  // Victim when the argmin does not run (static policy): the newest candidate,
  // i.e. the position leaving the window, or the decoded token when r = 0.
  __device__ int fixed_victim() const { return r > 0 ? ring_slot : kSelfVictim; }
  __device__ int fixed_victim_pos() const { return t - r; }
  // Logical row j: live ring slots [0, n_ring), then live heavy slots; row n_live is the new token.
  __device__ int slot_of(int j) const { return j < n_ring ? j : r + (j - n_ring); }
  __device__ bool is_cand(int s) const { return full && (s >= r || s == ring_slot); }
};

// Per-unit pointers.
template <typename GG>
struct UnitPtrs {
  char* K;
  char* V;
  const char* kn;
  const char* vn;
  const char* q;
  float* score;
  int32_t* pos;
  float* ks;
  float* vs;
  __device__ UnitPtrs(const DecodeArgs& a, int unit, int k) {
    const size_t ubase = (size_t)unit * k;
    K = (char*)a.k_slots + ubase * GG::ROWB;
    V = (char*)a.v_slots + ubase * GG::ROWB;
    kn = (const char*)a.k_new + (size_t)unit * GG::IROWB;
    vn = (const char*)a.v_new + (size_t)unit * GG::IROWB;
    q = (const char*)a.q + (size_t)unit * GG::IROWB;
    score = a.score + ubase;
    pos = a.pos + ubase;
    ks = GG::kQuant ? a.k_scale + ubase : nullptr;
    vs = GG::kQuant ? a.v_scale + ubase : nullptr;
  }
};

// The EPL input-row elements lane chunk c covers, as floats.
template <typename GG>
__device__ inline void load_input(const char* row, int c, float* x) {
#pragma unroll
  for (int i = 0; i < GG::ICH; ++i)
    GG::EI::unpack(load16(row + (c * GG::ICH + i) * 16), x + i * GG::EI::kPer16B);
}

// LDS stash of the rows the admission writes.
template <typename GG>
struct Stash {
  uint4 ring[2][GG::LPR];  // K, V of the ring slot leaving the window
  uint4 self[2][GG::LPR];  // K, V of the decoded token (cache format; not used for E4M3)
  float ring_scale[2];     // E4M3 row scales of the ring row
  // E4M3: the decoded token's K and V codes and row scales, computed where the
  // stream first reads its exact rows, for the admission at the end of the step
  uint4 tokq[2][GG::kQuant ? GG::LPR : 1];
  float tok_scale[2];
};

// E4M3 codes of a lane's 16 values of a row, and the row scale amax / 448 with
// amax taken over the lane's group of G lanes (lanes with act false hold no
// part of the row).
template <typename GG>
__device__ inline uint4 quantize_chunk(const float* x, bool act, float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < GG::EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = group_max<GG::G>(act ? amax : 0.f);
  scale = __fdiv_rn(amax, 448.f);
  return quantize16_e4m3(x, amax);
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4_t lds_v4;
typedef __attribute__((address_space(3))) float lds_f32;

__device__ inline uint4 lds_load16(const lds_char* p) {
  const u32x4_t v = *reinterpret_cast<const lds_v4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void lds_store16(lds_char* p, const uint4& x) {
  *reinterpret_cast<lds_v4*>(p) = u32x4_t{x.x, x.y, x.z, x.w};
}

// An admitted row's 16-byte chunk to the state buffers.
template <typename GG>
__device__ __forceinline__ void store_row(char* p, const uint4& v) {
  if constexpr (GG::kNtRows)
    store16_nt(p, v);
  else
    store16(p, v);
}

// The unit's K and V rows (and E4M3 row scales) held in LDS by the resident
// multi-step kernel: the same [k][row] layout as the state buffers.
template <typename GG>
struct ResRows {
  lds_char* K;
  lds_char* V;
  lds_f32* ks;   // E4M3 only
  lds_f32* vs;
};

// Inputs of one step (the lane's chunks of q and of the new token's K and V
// rows), loaded ahead of the step.
template <typename GG>
struct StepIn {
  uint4 q[GG::ICH];
  uint4 k[GG::ICH];
  uint4 v[GG::ICH];
};

// Uses the loaded registers of `in` here, so the compiler waits for their loads
// at this point rather than at their first later use.
template <typename GG>
__device__ __forceinline__ void settle(StepIn<GG>& in) {
  auto one = [](uint4& x) { asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w)); };
#pragma unroll
  for (int i = 0; i < GG::ICH; ++i) {
    one(in.q[i]);
    one(in.k[i]);
    one(in.v[i]);
  }
}

template <typename GG>
__device__ __forceinline__ void load_step_in(const UnitPtrs<GG>& u, int chunk, StepIn<GG>& in) {
#pragma unroll
  for (int i = 0; i < GG::ICH; ++i) {
    in.q[i] = load16(u.q + (chunk * GG::ICH + i) * 16);
    in.k[i] = load16(u.kn + (chunk * GG::ICH + i) * 16);
    in.v[i] = load16(u.vn + (chunk * GG::ICH + i) * 16);
  }
}

template <typename GG>
__device__ __forceinline__ void unpack_input(const uint4* c, float* x) {
#pragma unroll
  for (int i = 0; i < GG::ICH; ++i) GG::EI::unpack(c[i], x + i * GG::EI::kPer16B);
}

// Row batches base = lo, lo + NG, ... below hi, with the loads of DEPTH - 1
// batches in flight while one is consumed.  Loads are issued unconditionally,
// also for up to DEPTH - 1 batches past hi (the callers' fetch re-reads a valid
// row there), so every index into the register ring is a compile-time
// constant; consumption stops at the first batch past hi (a wave-uniform exit).
// `start` runs once the first batches are in flight, before any is consumed.
struct NoStart {
  __device__ void operator()() const {}
};
template <int DEPTH, int NG, typename Buf, typename F, typename C, typename S = NoStart>
__device__ __forceinline__ void row_pipeline(int lo, int hi, F&& fetch, C&& consume, S&& start = S{}) {
  Buf b[DEPTH];
#pragma unroll
  for (int i = 0; i + 1 < DEPTH; ++i) fetch(lo + i * NG, b[i]);
  start();
  for (int base = lo; base < hi; base += DEPTH * NG) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      if (base + i * NG >= hi) break;
      fetch(base + (i + DEPTH - 1) * NG, b[(i + DEPTH - 1) % DEPTH]);
      consume(base + i * NG, b[i]);
    }
  }
}

struct RowBuf {
  uint4 k, v;
};
struct QuantRowBuf {
  uint4 k, v;
  float ks, vs;
};

// Row batches in flight per wavefront.  With 8 wavefronts per workgroup the
// launch has few wavefronts per SIMD (few units, or a split over few units),
// so each keeps three batches of loads in flight; otherwise one.
template <typename GG>
constexpr int stream_depth() { return GG::NT / 64 >= 8 ? 4 : 2; }

// Streams logical rows [lo, hi): logit of each row into s_logit[j] (log2
// domain), per-row-group online softmax into (m, lsum, o).  The rows the
// admission writes are copied into the LDS stash when they fall in the range.
// Loads are unconditional (rows outside the range and idle lanes re-read a
// valid row and are masked out) so the compiler tracks outstanding loads
// exactly; the next row batch is in flight while the current one is consumed.
// With RES the cached rows come from the LDS copy `res` and the new token's
// rows from `in` (loaded ahead of the step); else both from global memory.
template <typename GG, int DEPTH = stream_depth<GG>(), bool RES = false>
__device__ __forceinline__ void stream_rows(const StepView& v, const UnitPtrs<GG>& u, int lo, int hi,
                                            const float* qf, float scale_log2, float* s_logit,
                                            Stash<GG>* st, float& m, float& lsum, float* o,
                                            const ResRows<GG>* res = nullptr, const StepIn<GG>* in = nullptr) {
  using EC = typename GG::EC;
  constexpr int EPL = GG::EPL, G = GG::G, RW = GG::RW, NG = GG::NG, LPR = GG::LPR;
  const int lane = threadIdx.x & 63;
  const int gl = lane & (G - 1);
  const int grp = (threadIdx.x >> 6) * RW + lane / G;
  const bool act = gl < LPR;
  const int chunk = act ? gl : 0;

  if constexpr (!GG::kQuant) {
    auto fetch = [&](int base, RowBuf& b) {
      const int j = base + grp;
      if constexpr (RES) {
        // LDS row k holds the decoded token; it also stands in past the range
        const int off = ((j < v.n_live && j < hi) ? v.slot_of(j) : v.k) * GG::ROWB + chunk * 16;
        b.k = lds_load16(res->K + off);
        b.v = lds_load16(res->V + off);
      } else {
        const char* kp = u.kn;
        const char* vp = u.vn;
        if (j < v.n_live && j < hi) {
          const size_t off = (size_t)v.slot_of(j) * GG::ROWB;
          kp = u.K + off;
          vp = u.V + off;
        }
        b.k = load16_stream(kp + chunk * 16);
        b.v = load16_stream(vp + chunk * 16);
      }
    };
    auto consume = [&](int base, const RowBuf& b) {
      const uint4& kr = b.k;
      const uint4& vr = b.v;
      float kf[EPL];
      EC::unpack(kr, kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qf[e], kf[e], d);  // qf is 0 on idle lanes
      d = group_sum<G>(d);
      const int j = base + grp;
      const bool valid = j < hi;
      const float lg = valid ? d * scale_log2 : -INFINITY;
      if (valid) {
        if (gl == 0) s_logit[j] = lg;
        if constexpr (!RES) {  // the resident rows stay readable in LDS until the admission
          if (act) {
            if (j == v.n_live) {
              st->self[0][gl] = kr;
              st->self[1][gl] = vr;
            } else if (v.ring_live && j == v.ring_slot) {
              st->ring[0][gl] = kr;
              st->ring[1][gl] = vr;
            }
          }
        }
      }
      if (lg > m + kLazyMax) {  // rare after the first rows: rescale to the new maximum
        const float alpha = fast_exp2(m - lg);  // 0 while m is kNoMax
        lsum *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
        m = lg;
      }
      const float p = fast_exp2(lg - m);  // 0 for rows outside the range; at most 2^kLazyMax
      float vf[EPL];
      EC::unpack(vr, vf);
      lsum += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e]);
    };
    row_pipeline<DEPTH, NG, RowBuf>(lo, hi, fetch, consume);
  } else {
    // The decoded token (exact bf16 row) seeds row group 0 when it is in range.
    // Its rows are loaded with the first row batch, and the seed runs while that
    // batch is in flight; its arithmetic is unconditional (results kept by a
    // select), so the loads stay ahead of every wait.
    const bool seed = v.n_live >= lo && v.n_live < hi;  // uniform
    uint4 tkr[GG::ICH], tvr[GG::ICH];
    if constexpr (!RES) {
#pragma unroll
      for (int i = 0; i < GG::ICH; ++i) {
        tkr[i] = load16(u.kn + (chunk * GG::ICH + i) * 16);
        tvr[i] = load16(u.vn + (chunk * GG::ICH + i) * 16);
      }
    }
    auto seed_group0 = [&]() __attribute__((always_inline)) {
      float kx[EPL], vx[EPL];
      if constexpr (RES) {
        unpack_input<GG>(in->k, kx);
        unpack_input<GG>(in->v, vx);
      } else {
        unpack_input<GG>(tkr, kx);
        unpack_input<GG>(tvr, vx);
      }
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qf[e], kx[e], d);
      d = group_sum<G>(d);
      const float ls = d * scale_log2;
      const bool own = seed && grp == 0;
      if (own && gl == 0) s_logit[v.n_live] = ls;
      // The token's codes for the admission, while the first batch is in
      // flight: every row group holds both rows; groups 0 and 1 (lanes [0, G)
      // and [G, 2G) of wave 0) quantize K and V.
      if (seed && threadIdx.x < 64) {  // uniform
        const int w = grp == 1 ? 1 : 0;
        float sc;
        const uint4 codes = quantize_chunk<GG>(w ? vx : kx, act, sc);
        if (grp < 2) {
          if (act) st->tokq[w][chunk] = codes;
          if (gl == 0) st->tok_scale[w] = sc;
        }
      }
      m = own ? ls : m;
      lsum = own ? 1.f : lsum;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = own ? (act ? vx[e] : 0.f) : o[e];
    };
    const int end = min(hi, v.n_live);  // cached rows only
    auto fetch = [&](int base, QuantRowBuf& b) {
      const int j = base + grp;
      const int s = (j < end) ? v.slot_of(j) : 0;  // slot 0 stands in past the end
      if constexpr (RES) {
        const int off = s * GG::ROWB + chunk * 16;
        b.k = lds_load16(res->K + off);
        b.v = lds_load16(res->V + off);
        b.ks = res->ks[s];
        b.vs = res->vs[s];
      } else {
        const size_t off = (size_t)s * GG::ROWB;
        b.k = load16_stream(u.K + off + chunk * 16);
        b.v = load16_stream(u.V + off + chunk * 16);
        b.ks = u.ks[s];
        b.vs = u.vs[s];
      }
    };
    auto consume = [&](int base, const QuantRowBuf& b) {
      const uint4& kr = b.k;
      const uint4& vr = b.v;
      const float ksc = b.ks;
      const float vsc = b.vs;
      float kf[EPL];
      EC::unpack(kr, kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qf[e], kf[e], d);
      d = group_sum<G>(d);
      const int j = base + grp;
      const bool valid = j < end;
      const float lg = valid ? d * ksc * scale_log2 : -INFINITY;
      if (valid) {
        if (gl == 0) s_logit[j] = lg;
        if constexpr (!RES) {
          if (v.ring_live && j == v.ring_slot) {
            if (act) {
              st->ring[0][gl] = kr;
              st->ring[1][gl] = vr;
            }
            if (gl == 0) {
              st->ring_scale[0] = ksc;
              st->ring_scale[1] = vsc;
            }
          }
        }
      }
      if (lg > m + kLazyMax) {  // rare after the first rows: rescale to the new maximum
        const float alpha = fast_exp2(m - lg);  // 0 while m is kNoMax
        lsum *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] *= alpha;
        m = lg;
      }
      const float p = fast_exp2(lg - m);  // 0 for rows outside the range
      const float pv = p * vsc;
      float vf[EPL];
      EC::unpack(vr, vf);
      lsum += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pv, vf[e], o[e]);
    };
    row_pipeline<DEPTH, NG, QuantRowBuf>(lo, end, fetch, consume, seed_group0);
  }
}

// Workgroup merge of the row groups: leaves M (block max), the group weights
// and L (block sum) in registers of every thread; s_o keeps the group outputs.
template <int NG>
struct GroupMerge {
  float M, L;
  float wg[NG];
};

template <typename GG, int D>
__device__ __forceinline__ GroupMerge<GG::NG> merge_groups(float m, float lsum, const float* o,
                                                           float (*s_o)[D], float* s_m, float* s_l) {
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
  GroupMerge<NG> r;
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

// The decoded token's K and V rows into slot `slot` of an E4M3 cache.
// STASHED: the codes and row scales wait in the LDS stash (computed where the
// stream first read the token); else lanes [0, G) of wave 0 quantize K and
// lanes [G, 2G) V from the exact rows in memory.  With RES the codes and
// scales also go to the LDS copy of the rows.
template <typename GG, bool RES = false, bool STASHED = true>
__device__ inline void admit_quantized(const UnitPtrs<GG>& u, int slot, const ResRows<GG>* res,
                                       const Stash<GG>* st) {
  constexpr int G = GG::G, LPR = GG::LPR, EPL = GG::EPL, ROWB = GG::ROWB;
  const int tid = threadIdx.x;
  if constexpr (STASHED) {
    if (tid < LPR) {
      const uint4 kc = st->tokq[0][tid];
      const uint4 vc = st->tokq[1][tid];
      store_row<GG>(u.K + (size_t)slot * ROWB + tid * 16, kc);
      store_row<GG>(u.V + (size_t)slot * ROWB + tid * 16, vc);
      if constexpr (RES) {
        lds_store16(res->K + slot * ROWB + tid * 16, kc);
        lds_store16(res->V + slot * ROWB + tid * 16, vc);
      }
    }
    if (tid == 0) {
      const float ksc = st->tok_scale[0], vsc = st->tok_scale[1];
      u.ks[slot] = ksc;
      u.vs[slot] = vsc;
      if constexpr (RES) {
        res->ks[slot] = ksc;
        res->vs[slot] = vsc;
      }
    }
  } else {
    if (tid >= 2 * G) return;
    const bool is_v = tid >= G;
    const int c = tid & (G - 1);
    const bool act = c < LPR;
    float x[EPL];
    load_input<GG>(is_v ? u.vn : u.kn, act ? c : 0, x);
    float sc;
    const uint4 codes = quantize_chunk<GG>(x, act, sc);
    if (act) store_row<GG>((is_v ? u.V : u.K) + (size_t)slot * ROWB + c * 16, codes);
    if (c == 0) (is_v ? u.vs : u.ks)[slot] = sc;
    if constexpr (RES) {
      if (act) lds_store16((is_v ? res->V : res->K) + slot * ROWB + c * 16, codes);
      if (c == 0) (is_v ? res->vs : res->ks)[slot] = sc;
    }
  }
}

// Score update, eviction argmin and admission for one unit, given the exact
// softmax max M and 1/L.  Logits of rows [0, n_att) are in s_logit; the
// scores this thread owns were prefetched into sc_pf / ps_pf; the ring row and
// the new token's row (E4M3: its codes and scales) are in the LDS stash.
// TOK_STASHED: the stream of this workgroup read the decoded token's rows and
// stashed them; the split kernel's combining workgroup may not have, and reads
// them from memory.
// SL: the scores and positions are in LDS (u.score / u.pos point there) and
// are read where they are used instead of being prefetched.
template <typename GG, bool RES = false, bool TOK_STASHED = true, bool SL = false>
__device__ __forceinline__ void finish_step(const StepView& v, const UnitPtrs<GG>& u, float M,
                                            float invL, float* s_logit, const float* sc_pf,
                                            const int* ps_pf, const Stash<GG>* st,
                                            unsigned long long* s_key, int* s_slot,
                                            int32_t* evicted, int unit, const ResRows<GG>* res = nullptr,
                                            const StepIn<GG>* in = nullptr) {
  constexpr int NT = GG::NT, PF = GG::PF, LPR = GG::LPR, ROWB = GG::ROWB;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float p_self = fast_exp2(s_logit[v.n_live] - M) * invL;
  const bool naive = v.policy == 2;      // score = this step's weight
  const bool argmin = v.policy != 1;     // static: fixed victim

  unsigned long long best = ~0ull;
  int best_slot = -1;
  if (v.r == 0 && tid == 0) {  // no window: the decoded token competes too
    best = ((unsigned long long)__float_as_uint(p_self) << 32) | (uint32_t)v.t;
    best_slot = kSelfVictim;
  }
  auto update = [&](int j, float lg, float old, int ps) {
    const int s = v.slot_of(j);
    const float ns = (naive ? 0.f : old) + fast_exp2(lg - M) * invL;
    s_logit[j] = ns;
    if (v.is_cand(s)) {
      const unsigned long long key = ((unsigned long long)__float_as_uint(ns) << 32) | (uint32_t)ps;
      if (key < best) {
        best = key;
        best_slot = s;
      }
    }
    return ns;
  };
  // The prefetched slots, without per-lane branches (every wavefront runs this
  // tail at once when the units stream in lockstep): all logits are read before
  // any new score is written back, so the LDS reads are in flight together;
  // lanes past n_live read the token's logit and stay out of the argmin.  When
  // every round has a live slot the rounds form one basic block; otherwise the
  // rounds past n_live are skipped by a uniform test.  The new scores stay in
  // registers for the stores below; only the ring row's goes to LDS, where
  // thread 0 reads it for the row leaving the window.
  float ns_pf[PF];
  float ring_ns = 0.f;
  auto pf_rounds = [&](auto all_live) __attribute__((always_inline)) {
    constexpr bool kAll = decltype(all_live)::value;
#pragma unroll
    for (int i = 0; i < PF; ++i)
      ns_pf[i] = kAll || i * NT < v.n_live ? s_logit[min(tid + i * NT, v.n_live)] : 0.f;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (!kAll && i * NT >= v.n_live) break;  // uniform
      const int j = tid + i * NT;
      const bool live = j < v.n_live;
      const int s = v.slot_of(j);
      const bool cand = live && v.is_cand(s);
      const float ns = (naive ? 0.f : sc_pf[i]) + fast_exp2(ns_pf[i] - M) * invL;
      ns_pf[i] = ns;
      ring_ns = j == v.ring_slot ? ns : ring_ns;
      const unsigned long long key = ((unsigned long long)__float_as_uint(ns) << 32) | (uint32_t)ps_pf[i];
      const bool take = cand && key < best;
      best = take ? key : best;
      best_slot = take ? s : best_slot;
    }
  };
  if constexpr (SL) {
    // Scores and positions in LDS (multi-step kernels), read per live slot:
    // there the tail of one unit overlaps the streaming of others.  Rounds
    // past the live slots are skipped by a uniform test.
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (i * NT >= v.n_live) break;  // uniform
      const int j = tid + i * NT;
      ns_pf[i] = j < v.n_live ? s_logit[j] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (i * NT >= v.n_live) break;  // uniform
      const int j = tid + i * NT;
      if (j < v.n_live) {
        const int s = v.slot_of(j);
        ns_pf[i] = update(j, ns_pf[i], u.score[s], v.is_cand(s) ? u.pos[s] : 0);
      }
    }
  } else if (v.n_live > (PF - 1) * NT) {
    pf_rounds(std::true_type{});
  } else {
    pf_rounds(std::false_type{});
  }
  if (!SL && v.ring_slot >= 0 && v.ring_slot < v.n_live && v.ring_slot < PF * NT && v.ring_slot % NT == tid)
    s_logit[v.ring_slot] = ring_ns;
  // Slots past the prefetched ones (budgets above PF * NT): their scores and
  // positions are loaded kRest at a time before any is used, one memory round
  // trip per batch instead of per slot (the argmin over unique keys does not
  // depend on the order).
  constexpr int kRest = 8;
  for (int j0 = tid + PF * NT; j0 < v.n_live; j0 += kRest * NT) {
    float old[kRest];
    int ps[kRest];
#pragma unroll
    for (int i = 0; i < kRest; ++i) {
      const int s = v.slot_of(min(j0 + i * NT, v.n_live - 1));
      old[i] = u.score[s];
      ps[i] = u.pos[s];  // used for candidates only
    }
#pragma unroll
    for (int i = 0; i < kRest; ++i) {
      const int j = j0 + i * NT;
      if (j < v.n_live) update(j, s_logit[j], old[i], ps[i]);
    }
  }

  // The victim's key and slot: each wavefront's minimum and the slot of the
  // lane holding it go to LDS, and after one barrier every thread takes the
  // smallest (keys are unique: positions differ).
  unsigned long long vkey = ~0ull;
  int victim = v.fixed_victim();
  if (v.full && !argmin) {
    vkey = (uint32_t)v.fixed_victim_pos();
  } else if (v.full) {
    const unsigned long long w = wave_min_u64(best);
    if (lane == 0) s_key[wave] = w;
    if (best_slot != -1 && best == w) s_slot[wave] = best_slot;
    __syncthreads();
    int wi = 0;
    vkey = s_key[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      const unsigned long long ki = s_key[i];
      if (ki < vkey) {
        vkey = ki;
        wi = i;
      }
    }
    victim = s_slot[wi];
  } else if (!v.full) {
    __syncthreads();  // thread 0 reads the updated score of the ring row below
  }

  // dst: where the row leaving the window goes (the victim's heavy slot, or the
  // next free heavy slot while the cache is not yet full; -1 if it is dropped or
  // still inside the window).  adm: where the decoded token goes (its ring slot;
  // with r = 0 the victim's slot or the next free one, -1 if it is the victim).
  int dst = -1, adm;
  if (v.r > 0) {
    adm = v.ring_slot;
    if (v.full) {
      if (victim != v.ring_slot) dst = victim;
    } else if (v.ring_live) {
      dst = v.r + v.n_heavy;
    }
  } else {
    adm = v.full ? (victim == kSelfVictim ? -1 : victim) : v.n_live;
  }

  auto write_score = [&](int j, float ns) {
    const int s = v.slot_of(j);
    if (s != adm && s != dst) u.score[s] = ns;
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    if (i * NT >= v.n_live) break;  // uniform
    const int j = tid + i * NT;
    if (j < v.n_live) write_score(j, ns_pf[i]);
  }
  for (int j = tid + PF * NT; j < v.n_live; j += NT) write_score(j, s_logit[j]);

  if (tid == 0) {
    if (dst >= 0) {
      u.score[dst] = s_logit[v.ring_slot];
      u.pos[dst] = v.t - v.r;
      if constexpr (GG::kQuant) {
        if constexpr (RES) {
          // read before the token's admission below (same wavefront) replaces them
          const float rk = res->ks[v.ring_slot], rv = res->vs[v.ring_slot];
          u.ks[dst] = rk;
          u.vs[dst] = rv;
          res->ks[dst] = rk;
          res->vs[dst] = rv;
        } else {
          u.ks[dst] = st->ring_scale[0];
          u.vs[dst] = st->ring_scale[1];
        }
      }
    }
    if (adm >= 0) {
      u.score[adm] = p_self;
      u.pos[adm] = v.t;
    }
    if (evicted) evicted[unit] = v.full ? (int32_t)(uint32_t)vkey : -1;
  }
  if constexpr (RES) {
    // Thread tid < LPR moves chunk tid of the rows: the ring row is read from
    // LDS before the token replaces it; the token's rows are LDS row k (their
    // codes in the stash for E4M3).
    if (tid < LPR && dst >= 0) {
      const uint4 rk = lds_load16(res->K + v.ring_slot * ROWB + tid * 16);
      const uint4 rv = lds_load16(res->V + v.ring_slot * ROWB + tid * 16);
      store_row<GG>(u.K + (size_t)dst * ROWB + tid * 16, rk);
      store_row<GG>(u.V + (size_t)dst * ROWB + tid * 16, rv);
      lds_store16(res->K + dst * ROWB + tid * 16, rk);
      lds_store16(res->V + dst * ROWB + tid * 16, rv);
    }
    if (adm >= 0) {
      if constexpr (GG::kQuant) {
        admit_quantized<GG, true, true>(u, adm, res, st);
      } else if (tid < LPR) {
        const uint4 tk = lds_load16(res->K + v.k * ROWB + tid * 16);
        const uint4 tv = lds_load16(res->V + v.k * ROWB + tid * 16);
        store_row<GG>(u.K + (size_t)adm * ROWB + tid * 16, tk);
        store_row<GG>(u.V + (size_t)adm * ROWB + tid * 16, tv);
        lds_store16(res->K + adm * ROWB + tid * 16, tk);
        lds_store16(res->V + adm * ROWB + tid * 16, tv);
      }
    }
  } else {
    if (tid < LPR && dst >= 0) {
      store_row<GG>(u.K + (size_t)dst * ROWB + tid * 16, st->ring[0][tid]);
      store_row<GG>(u.V + (size_t)dst * ROWB + tid * 16, st->ring[1][tid]);
    }
    if (adm >= 0) {
      if constexpr (GG::kQuant) {
        admit_quantized<GG, false, TOK_STASHED>(u, adm, nullptr, st);
      } else if (tid < LPR) {
        store_row<GG>(u.K + (size_t)adm * ROWB + tid * 16, st->self[0][tid]);
        store_row<GG>(u.V + (size_t)adm * ROWB + tid * 16, st->self[1][tid]);
      }
    }
  }
}

// Prefetch of the scores a thread will update, and of the candidates'
// positions.  With kAll the loads are unconditional (threads past the live
// slots read slot 0's score, threads of other slots slot 0's position, and
// ignore them), so they all go out at once and the compiler counts them
// exactly: the split decode's combining workgroup issues them that way with
// its partials' loads.  The per-step kernels measured slightly faster with
// guarded loads.
template <typename GG, bool kAll = false>
__device__ __forceinline__ void prefetch_scores(const StepView& v, const UnitPtrs<GG>& u, float* sc_pf,
                                                int* ps_pf) {
#pragma unroll
  for (int i = 0; i < GG::PF; ++i) {
    const int j = threadIdx.x + i * GG::NT;
    if constexpr (kAll) {
      const int s = j < v.n_live ? v.slot_of(j) : 0;
      sc_pf[i] = u.score[s];
      ps_pf[i] = u.pos[v.is_cand(s) ? s : 0];
    } else {
      sc_pf[i] = 0.f;
      ps_pf[i] = 0;
      if (j < v.n_live) {
        const int s = v.slot_of(j);
        sc_pf[i] = u.score[s];
        if (v.is_cand(s)) ps_pf[i] = u.pos[s];
      }
    }
  }
}

// Workgroup-shared state of one decode step.
template <typename GG, int D>
struct StepShared {
  float s_o[GG::NG][D];
  float s_m[GG::NG];
  float s_l[GG::NG];
  Stash<GG> st;
  unsigned long long s_key[GG::NT / 64];
  int s_slot[GG::NT / 64];
};

// One decode step of one unit by the whole workgroup.  s_logit: LDS, at least
// n_live + 1 floats.  score_lds / pos_lds: when not null, the unit's scores and
// positions live in LDS (k entries each) instead of the state buffers.
// With RES the cached rows are read from the LDS copy `res` (kept current by
// the admission) and the step's inputs come from `in`, which is not read after
// the row stream; `streamed` runs there.
template <typename GG, int D, bool RES = false, bool SL = false, typename H = NoStart>
__device__ __forceinline__ void unit_step(const DecodeArgs& a, int unit, StepShared<GG, D>& sh, float* s_logit,
                                          float* score_lds, int32_t* pos_lds, const ResRows<GG>* res = nullptr,
                                          const StepIn<GG>* in = nullptr, H&& streamed = H{}) {
  constexpr int EPL = GG::EPL, LPR = GG::LPR, NG = GG::NG, NT = GG::NT, PF = GG::PF;
  const int tid = threadIdx.x;
  const StepView v(a);
  UnitPtrs<GG> u(a, unit, v.k);
  if (score_lds) {
    u.score = score_lds;
    u.pos = pos_lds;
  }
  const int gl = (tid & 63) & (GG::G - 1);
  const bool act = gl < LPR;

  float qf[EPL];
  if constexpr (RES)
    unpack_input<GG>(in->q, qf);
  else
    load_input<GG>(u.q, act ? gl : 0, qf);
  if (!act) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[e] = 0.f;
  }
  float sc_pf[SL ? 1 : PF];
  int ps_pf[SL ? 1 : PF];
  if constexpr (!SL) prefetch_scores<GG>(v, u, sc_pf, ps_pf);

  float m = kNoMax, lsum = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  if constexpr (RES)
    stream_rows<GG, 2, true>(v, u, 0, v.n_att, qf, a.scale_log2, s_logit, &sh.st, m, lsum, o, res, in);
  else
    stream_rows<GG>(v, u, 0, v.n_att, qf, a.scale_log2, s_logit, &sh.st, m, lsum, o);
  streamed();

  const GroupMerge<NG> gm = merge_groups<GG, D>(m, lsum, o, sh.s_o, sh.s_m, sh.s_l);
  const float invL = 1.f / gm.L;
  // The persistent launches at large batch store the output with the
  // non-temporal hint: there one unit's stores go out while other units
  // stream their rows, and the hint made those steps 3-5% faster; with one
  // launch per step, or at small batch, it made them slower.
  constexpr bool kNtOut = SL && !RES && NT <= 256;
  for (int c = tid; c < D; c += NT) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc = fmaf(sh.s_o[g][c], gm.wg[g], acc);
    if constexpr (kNtOut)
      __builtin_nontemporal_store(acc * invL, a.out + (size_t)unit * D + c);
    else
      a.out[(size_t)unit * D + c] = acc * invL;
  }
  finish_step<GG, RES, true, SL>(v, u, gm.M, invL, s_logit, sc_pf, ps_pf, &sh.st, sh.s_key, sh.s_slot, a.evicted,
                                 unit, res, in);
}

template <typename T, typename C, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using GG = Geo<T, C, D, NW>;
  __shared__ StepShared<GG, D> sh;
  extern __shared__ float s_logit[];  // [n_live + 1] logits, later updated scores
  unit_step<GG, D>(a, blockIdx.x, sh, s_logit, nullptr, nullptr);
}

// n_steps consecutive steps over tokens known in advance, in one launch: each
// workgroup carries its unit from step to step, so one unit's score update and
// admission overlap other units' streaming, and the unit's scores and
// positions stay in LDS until the last step.  `a` describes the first step;
// live0 = live slots before it.  Inputs of step s start at s * units rows, as
// do the outputs.  Rows admitted at one step are read at the next by other
// threads of the same workgroup: the workgroup barrier between steps orders
// them.
// With up to four wavefronts per unit (more than 512 units), four waves per
// SIMD: a unit whose workgroup is not resident would wait for whole launches
// of the others (3584 single-wave units need 3.5 per SIMD, 1024 four-wave
// units 4).  Eight-wavefront units (small batches) are not bounded.
template <typename T, typename C, int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW <= 4 ? 4 : 1))) void decode_multi_kernel(
    DecodeArgs a, int n_steps, int live0) {
  using GG = Geo<T, C, D, NW>;
  __shared__ StepShared<GG, D> sh;
  extern __shared__ float dyn[];  // logits [k + 1], scores [k], positions [k]
  const int k = a.k;
  float* s_logit = dyn;
  float* s_score = dyn + k + 1;
  int32_t* s_pos = reinterpret_cast<int32_t*>(s_score + k);
  const int unit = blockIdx.x;
  const size_t ubase = (size_t)unit * k;
  for (int i = threadIdx.x; i < k; i += GG::NT) {
    s_score[i] = a.score[ubase + i];
    s_pos[i] = a.pos[ubase + i];
  }
  __syncthreads();
  const size_t in_step = (size_t)a.units * GG::IROWB;
  for (int st = 0; st < n_steps; ++st) {
    DecodeArgs as = a;
    as.t = a.t + st;
    const int n_live = min(live0 + st, k);
    as.n_ring = min(as.t, a.r);
    as.n_heavy = n_live - as.n_ring;
    as.q = (const char*)a.q + st * in_step;
    as.k_new = (const char*)a.k_new + st * in_step;
    as.v_new = (const char*)a.v_new + st * in_step;
    as.out = a.out + (size_t)st * a.units * D;
    as.evicted = a.evicted ? a.evicted + (size_t)st * a.units : nullptr;
    unit_step<GG, D, false, true>(as, unit, sh, s_logit, s_score, s_pos);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < k; i += GG::NT) {
    a.score[ubase + i] = s_score[i];
    a.pos[ubase + i] = s_pos[i];
  }
}

// n_steps consecutive steps with the unit's whole state in LDS: its K and V rows
// (and E4M3 row scales), scores and positions are read once at launch; a step
// streams the rows from LDS, and its admission writes the admitted rows both to
// LDS and to the state buffers; scores and positions go back at the end.  Each
// step's inputs (q and the new token's rows) are loaded during the step before.
// A workgroup holds 2k rows of LDS (k = 256, d = 128 bf16: 128 KB), so this
// runs when that fits the device's per-workgroup LDS and there are no more
// units than compute units.  Same arithmetic as decode_kernel, step for step.
template <typename T, typename C, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_resident_kernel(DecodeArgs a, int n_steps, int live0) {
  using GG = Geo<T, C, D, NW>;
  constexpr int ROWB = GG::ROWB, NT = GG::NT;
  __shared__ StepShared<GG, D> sh;
  extern __shared__ float dynr[];  // K rows, V rows, [K scales, V scales], logits [k + 1], scores [k], positions [k]
  const int k = a.k;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  // Unquantized caches keep one row more in K and V: row k holds the decoded
  // token, written at the end of the step before (the E4M3 path takes the
  // token's exact row from registers).
  constexpr int XR = GG::kQuant ? 0 : 1;
  lds_char* base = (lds_char*)dynr;
  ResRows<GG> res;
  res.K = base;
  res.V = base + (k + XR) * ROWB;
  res.ks = res.vs = nullptr;
  int words = 2 * (k + XR) * ROWB / 4;  // floats before the logits
  if constexpr (GG::kQuant) {
    res.ks = (lds_f32*)(base + 2 * k * ROWB);
    res.vs = res.ks + k;
    words += 2 * k;
  }
  float* s_logit = dynr + words;
  float* s_score = s_logit + k + 1;
  int32_t* s_pos = reinterpret_cast<int32_t*>(s_score + k);

  const size_t ubase = (size_t)unit * k;
  {
    // the unit's rows, four 16-byte loads of each tensor in flight per thread
    const char* Kg = (const char*)a.k_slots + ubase * ROWB;
    const char* Vg = (const char*)a.v_slots + ubase * ROWB;
    const int n16 = k * ROWB / 16;
    for (int i0 = tid; i0 < n16; i0 += 4 * NT) {
      uint4 kb[4], vb[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = min(i0 + w * NT, n16 - 1);
        kb[w] = load16(Kg + (size_t)i * 16);
        vb[w] = load16(Vg + (size_t)i * 16);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = i0 + w * NT;
        if (i < n16) {
          lds_store16(res.K + i * 16, kb[w]);
          lds_store16(res.V + i * 16, vb[w]);
        }
      }
    }
  }
  for (int i = tid; i < k; i += NT) {
    s_score[i] = a.score[ubase + i];
    s_pos[i] = a.pos[ubase + i];
    if constexpr (GG::kQuant) {
      res.ks[i] = a.k_scale[ubase + i];
      res.vs[i] = a.v_scale[ubase + i];
    }
  }
  const size_t in_step = (size_t)a.units * GG::IROWB;
  const int gl = (tid & 63) & (GG::G - 1);
  const int chunk = gl < GG::LPR ? gl : 0;
  StepIn<GG> cur, nxt;
  load_step_in<GG>(UnitPtrs<GG>(a, unit, k), chunk, cur);
  if constexpr (XR) {
    if (tid < GG::LPR) {
      lds_store16(res.K + k * ROWB + tid * 16, cur.k[0]);
      lds_store16(res.V + k * ROWB + tid * 16, cur.v[0]);
    }
  }
  __syncthreads();
  for (int st = 0; st < n_steps; ++st) {
    DecodeArgs as = a;
    as.t = a.t + st;
    const int n_live = min(live0 + st, k);
    as.n_ring = min(as.t, a.r);
    as.n_heavy = n_live - as.n_ring;
    as.q = (const char*)a.q + st * in_step;
    as.k_new = (const char*)a.k_new + st * in_step;
    as.v_new = (const char*)a.v_new + st * in_step;
    as.out = a.out + (size_t)st * a.units * D;
    as.evicted = a.evicted ? a.evicted + (size_t)st * a.units : nullptr;
    const bool more = st + 1 < n_steps;
    {
      // the next step's inputs (the last step re-reads its own: every path loads)
      const size_t adv = more ? in_step : 0;
      DecodeArgs an = as;
      an.q = (const char*)as.q + adv;
      an.k_new = (const char*)as.k_new + adv;
      an.v_new = (const char*)as.v_new + adv;
      load_step_in<GG>(UnitPtrs<GG>(an, unit, k), chunk, nxt);
    }
    // They move into `cur` once this step's rows are streamed, long after their
    // loads arrived; left to the first use at the end of the step, the wait
    // for them would also wait for the acknowledgement of the step's stores.
    unit_step<GG, D, true, true>(as, unit, sh, s_logit, s_score, s_pos, &res, &cur, [&]() {
      settle(nxt);
      cur = nxt;
    });
    if constexpr (XR) {
      // the next token's row; every read of row k in this step (the stream, and
      // the admission by these same threads) comes before
      if (more && tid < GG::LPR) {
        lds_store16(res.K + k * ROWB + tid * 16, cur.k[0]);
        lds_store16(res.V + k * ROWB + tid * 16, cur.v[0]);
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < k; i += NT) {
    a.score[ubase + i] = s_score[i];
    a.pos[ubase + i] = s_pos[i];
  }
}

// Device-scope (agent) relaxed store and load: global_store / global_load with
// sc1 on gfx950, coherent across the XCDs without a cache writeback.
__device__ __forceinline__ void publish(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float collect(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, typename C, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(DecodeArgs a, SplitScratch sp) {
  using GG = Geo<T, C, D, NW>;
  constexpr int EPL = GG::EPL, LPR = GG::LPR, NG = GG::NG, NT = GG::NT, PF = GG::PF;
  constexpr int ROWB = GG::ROWB;

  __shared__ float s_o[NG][D];
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];
  __shared__ Stash<GG> st;
  __shared__ unsigned long long s_key[NW];
  __shared__ int s_slot[NW];
  __shared__ int s_last;
  extern __shared__ float s_logit[];  // [n_live + 1]

  const int S = sp.splits;
  const int unit = blockIdx.x / S;
  const int part = blockIdx.x % S;
  const int tid = threadIdx.x;
  const StepView v(a);
  const UnitPtrs<GG> u(a, unit, v.k);
  const int gl = (tid & 63) & (GG::G - 1);
  const bool act = gl < LPR;

  float qf[EPL];
  load_input<GG>(u.q, act ? gl : 0, qf);
  if (!act) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[e] = 0.f;
  }
  const int per = (v.n_att + S - 1) / S;
  const int lo = min(v.n_att, part * per);
  const int hi = min(v.n_att, lo + per);
  float m = kNoMax, lsum = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  stream_rows<GG>(v, u, lo, hi, qf, a.scale_log2, s_logit, &st, m, lsum, o);
  const GroupMerge<NG> gm = merge_groups<GG, D>(m, lsum, o, s_o, s_m, s_l);

  // This workgroup's partial: max, sum, output relative to its max; its logits.
  // Device-scope stores (sc1): each is written through to the level that all
  // XCDs share, so no cache of this XCD has to be written back for the
  // combining workgroup (possibly on another XCD) to read it.
  float* pp = sp.partials + ((size_t)unit * S + part) * (D + 2);
  if (tid == 0) {
    publish(pp + 0, gm.M);
    publish(pp + 1, gm.L);
  }
  for (int c = tid; c < D; c += NT) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc = fmaf(s_o[g][c], gm.wg[g], acc);
    publish(pp + 2 + c, acc);
  }
  float* lg = sp.logits + (size_t)unit * (v.k + 1);
  for (int j = lo + tid; j < hi; j += NT) publish(lg + j, s_logit[j]);

  // Count arrivals; the last workgroup of the unit finishes the step.  Every
  // thread waits until its device-scope stores are acknowledged before the
  // barrier, so when thread 0 counts the arrival all of the workgroup's
  // partials are visible at device scope; the combining workgroup reads them
  // with device-scope loads after it has seen the final count.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(sp.counters + unit, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Combine the partials.  Loads are issued in batches of kBatch before any
  // of them is used, so the combine costs a few memory round trips instead of
  // one per partial and per logit; sums keep the order c = 0, 1, ..., S - 1.
  // The partials' maxima and sums (S <= 64 each) live in s_o, free once this
  // workgroup's own partial is published: the kernel takes no more LDS than
  // the fused one, as the launch-time LDS check assumes.
  static_assert(NG * D >= 128, "s_o holds the partials' maxima and sums");
  float* s_pm = &s_o[0][0];
  float* s_pl = s_pm + 64;
  constexpr int kBatch = 8;
  const float* up = sp.partials + (size_t)unit * S * (D + 2);
  // Only this workgroup updates the scores: their loads start here, in flight
  // with the partials'.
  float sc_pf[PF];
  int ps_pf[PF];
  prefetch_scores<GG, true>(v, u, sc_pf, ps_pf);
  // The rows the admission writes (still intact: only this workgroup writes
  // the unit's state) and the partials' maxima and sums go into registers
  // first, in flight with the logits, and into LDS after them.
  uint4 row[4] = {};  // K, V of the decoded token (unquantized caches), K, V of the ring row
  float ring_sc[2] = {0.f, 0.f};
  if (tid < LPR) {
    if constexpr (!GG::kQuant) {
      row[0] = load16(u.kn + tid * 16);
      row[1] = load16(u.vn + tid * 16);
    }
    if (v.ring_live) {
      row[2] = load16(u.K + (size_t)v.ring_slot * ROWB + tid * 16);
      row[3] = load16(u.V + (size_t)v.ring_slot * ROWB + tid * 16);
    }
  }
  if constexpr (GG::kQuant) {
    if (tid == 0 && v.ring_live) {
      ring_sc[0] = u.ks[v.ring_slot];
      ring_sc[1] = u.vs[v.ring_slot];
    }
  }
  float pm = 0.f, pl = 0.f;
  if (tid < S) {
    pm = collect(up + (size_t)tid * (D + 2));
    pl = collect(up + (size_t)tid * (D + 2) + 1);
  }
  // The first kBatch partials' outputs of column tid, in flight with the rest.
  float ov0[kBatch];
  if (tid < D) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) ov0[i] = collect(up + (size_t)min(i, S - 1) * (D + 2) + 2 + tid);
  }
  // All logits (indices clamped to the last one; only those below n_att are
  // kept), kLogits per thread per round: the k + 1 logits of a budget k up to
  // kLogits * NT - 1 (4607 with 8 wavefronts) take one round trip.
  constexpr int kLogits = kBatch + 1;
  for (int j0 = tid; j0 < v.n_att; j0 += kLogits * NT) {
    float lv[kLogits];
#pragma unroll
    for (int i = 0; i < kLogits; ++i) lv[i] = collect(lg + min(j0 + i * NT, v.n_att - 1));
#pragma unroll
    for (int i = 0; i < kLogits; ++i)
      if (j0 + i * NT < v.n_att) s_logit[j0 + i * NT] = lv[i];
  }
  if (tid < S) {
    s_pm[tid] = pm;
    s_pl[tid] = pl;
  }
  if (tid < LPR) {
    if constexpr (!GG::kQuant) {
      st.self[0][tid] = row[0];
      st.self[1][tid] = row[1];
    }
    if (v.ring_live) {
      st.ring[0][tid] = row[2];
      st.ring[1][tid] = row[3];
    }
  }
  if constexpr (GG::kQuant) {
    if (tid == 0 && v.ring_live) {
      st.ring_scale[0] = ring_sc[0];
      st.ring_scale[1] = ring_sc[1];
    }
  }
  __syncthreads();
  float M = -INFINITY;
  for (int c = 0; c < S; ++c) M = fmaxf(M, s_pm[c]);
  float L = 0.f;
  for (int c = 0; c < S; ++c) L = fmaf(s_pl[c], fast_exp2(s_pm[c] - M), L);
  const float invL = 1.f / L;
  for (int d = tid; d < D; d += NT) {
    float acc = 0.f;
    for (int c0 = 0; c0 < S; c0 += kBatch) {
      float ov[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        ov[i] = d == tid && c0 == 0 ? ov0[i] : collect(up + (size_t)min(c0 + i, S - 1) * (D + 2) + 2 + d);
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (c0 + i < S) acc = fmaf(ov[i], fast_exp2(s_pm[c0 + i] - M), acc);
    }
    a.out[(size_t)unit * D + d] = acc * invL;
  }
  __syncthreads();
  finish_step<GG, false, false>(v, u, M, invL, s_logit, sc_pf, ps_pf, &st, s_key, s_slot, a.evicted, unit);
  if (tid == 0) sp.counters[unit] = 0u;  // ready for the next step
}

// Dynamic LDS of the resident kernel: rows, E4M3 row scales, logits, scores, positions.
template <typename T, typename C, int D>
size_t resident_dyn_lds(int k) {
  constexpr bool quant = std::is_same<C, e4m3>::value;
  const size_t rows = quant ? (size_t)k : (size_t)k + 1;  // unquantized: one more row for the token
  return 2 * rows * D * Elem<C>::kBytes + (quant ? (size_t)8 * k : 0) + (size_t)(3 * k + 1) * sizeof(float);
}

template <typename T, typename C, int D, int NW>
hipError_t launch_multi_nw(const DecodeArgs& a, int n_steps, int live0, bool resident, hipStream_t s) {
  if (resident) {
    const size_t lds = resident_dyn_lds<T, C, D>(a.k);
    const hipError_t e = hipFuncSetAttribute((const void*)decode_resident_kernel<T, C, D, NW>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_resident_kernel<T, C, D, NW>), dim3(a.units), dim3(NW * 64), lds, s, a, n_steps,
                       live0);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(3 * a.k + 1) * sizeof(float);
  hipLaunchKernelGGL((decode_multi_kernel<T, C, D, NW>), dim3(a.units), dim3(NW * 64), lds, s, a, n_steps,
                     live0);
  return hipGetLastError();
}

template <typename T, typename C, int D, int NW>
int multi_per_cu_nw(int k) {
  int n = 0;
  const size_t lds = (size_t)(3 * k + 1) * sizeof(float);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_multi_kernel<T, C, D, NW>, NW * 64, lds) !=
      hipSuccess)
    return 0;
  return n;
}

template <typename T, typename C, int D>
int multi_per_cu_d(int k, int waves) {
  switch (waves) {
    case 1: return multi_per_cu_nw<T, C, D, 1>(k);
    case 2: return multi_per_cu_nw<T, C, D, 2>(k);
    case 4: return multi_per_cu_nw<T, C, D, 4>(k);
    case 8: return multi_per_cu_nw<T, C, D, 8>(k);
    default: return 0;
  }
}

template <typename T, typename C>
int multi_per_cu_t(int k, int head_dim, int waves) {
  switch (head_dim) {
    case 64: return multi_per_cu_d<T, C, 64>(k, waves);
    case 96: return multi_per_cu_d<T, C, 96>(k, waves);
    case 128: return multi_per_cu_d<T, C, 128>(k, waves);
    default: return 0;
  }
}

template <typename T, typename C, int D>
hipError_t launch_multi_d(const DecodeArgs& a, int waves, int n_steps, int live0, bool resident, hipStream_t s) {
  switch (waves) {
    case 1: return launch_multi_nw<T, C, D, 1>(a, n_steps, live0, resident, s);
    case 2: return launch_multi_nw<T, C, D, 2>(a, n_steps, live0, resident, s);
    case 4: return launch_multi_nw<T, C, D, 4>(a, n_steps, live0, resident, s);
    case 8: return launch_multi_nw<T, C, D, 8>(a, n_steps, live0, resident, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename C>
hipError_t launch_multi_t(const DecodeArgs& a, int head_dim, int waves, int n_steps, int live0, bool resident,
                          hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_multi_d<T, C, 64>(a, waves, n_steps, live0, resident, s);
    case 96: return launch_multi_d<T, C, 96>(a, waves, n_steps, live0, resident, s);
    case 128: return launch_multi_d<T, C, 128>(a, waves, n_steps, live0, resident, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename C>
size_t resident_dyn_lds_t(int k, int head_dim) {
  switch (head_dim) {
    case 64: return resident_dyn_lds<T, C, 64>(k);
    case 96: return resident_dyn_lds<T, C, 96>(k);
    case 128: return resident_dyn_lds<T, C, 128>(k);
    default: return (size_t)-1 / 2;
  }
}

template <typename T, typename C, int D, int NW>
hipError_t launch_nw(const DecodeArgs& a, const SplitScratch* sp, hipStream_t s) {
  const int n_live = a.n_ring + a.n_heavy;
  const size_t lds = (size_t)(n_live + 1) * sizeof(float);
  if (sp && sp->splits > 1) {
    hipLaunchKernelGGL((decode_split_kernel<T, C, D, NW>), dim3(a.units * sp->splits),
                       dim3(NW * 64), lds, s, a, *sp);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, C, D, NW>), dim3(a.units), dim3(NW * 64), lds, s, a);
  }
  return hipGetLastError();
}

template <typename T, typename C, int D>
hipError_t launch_d(const DecodeArgs& a, int waves, const SplitScratch* sp, hipStream_t s) {
  switch (waves) {
    case 1: return launch_nw<T, C, D, 1>(a, sp, s);
    case 2: return launch_nw<T, C, D, 2>(a, sp, s);
    case 4: return launch_nw<T, C, D, 4>(a, sp, s);
    case 8: return launch_nw<T, C, D, 8>(a, sp, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename C>
hipError_t launch_t(const DecodeArgs& a, int head_dim, int waves, const SplitScratch* sp,
                    hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<T, C, 64>(a, waves, sp, s);
    case 96: return launch_d<T, C, 96>(a, waves, sp, s);
    case 128: return launch_d<T, C, 128>(a, waves, sp, s);
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

int decode_split_auto(int units, int waves, int k, int cus) {
  // One workgroup per unit, unless the units leave compute units idle, the
  // budget is at least kMinK and each share still streams at least kMinRows
  // rows.  Measured on MI355X (32 units, 8 wavefronts per workgroup): 8 shares
  // of 512 or 1024 rows ran 2.6x and 3.0x faster than one workgroup per unit,
  // 4 shares of 256 rows 1.24x and 3 shares of 256 rows 1.07x; 2 shares of 256
  // rows (k = 512) and shares of 128 rows lost, the publication round trips
  // (store acknowledgement, arrival count, reads of the partials) costing more
  // than the streaming they save.
  constexpr int kMinRows = 256;
  constexpr int kMinK = 768;
  if (waves < 8 || units >= cus || k < kMinK) return 1;
  int s = cus / units;
  if (s > k / kMinRows) s = k / kMinRows;
  if (s > 64) s = 64;
  return s < 1 ? 1 : s;
}

namespace {

template <typename T, typename C>
size_t static_lds_t(int head_dim, int waves) {
  switch (head_dim * 16 + waves) {
#define H2O_LDS_CASE(D, NW) \
  case D * 16 + NW: return sizeof(StepShared<Geo<T, C, D, NW>, D>) + 64;
    H2O_LDS_CASE(64, 1) H2O_LDS_CASE(64, 2) H2O_LDS_CASE(64, 4) H2O_LDS_CASE(64, 8)
    H2O_LDS_CASE(96, 1) H2O_LDS_CASE(96, 2) H2O_LDS_CASE(96, 4) H2O_LDS_CASE(96, 8)
    H2O_LDS_CASE(128, 1) H2O_LDS_CASE(128, 2) H2O_LDS_CASE(128, 4) H2O_LDS_CASE(128, 8)
#undef H2O_LDS_CASE
    default: return kMaxLds + 1;  // no such instantiation: never fits
  }
}

}  // namespace

size_t decode_static_lds(int dtype, int cache, int head_dim, int waves) {
  // the split kernel holds the same arrays plus one int (the 64-byte margin)
  if (cache == 1) return static_lds_t<bf16, e4m3>(head_dim, waves);
  if (dtype == 0) return static_lds_t<float, float>(head_dim, waves);
  return static_lds_t<bf16, bf16>(head_dim, waves);
}

bool decode_multi_fits(int k, int dtype, int cache, int head_dim, int waves) {
  // logits, scores and positions of the unit in LDS: 3k + 1 words
  return decode_static_lds(dtype, cache, head_dim, waves) + (size_t)(3 * k + 1) * 4 <= kMaxLds;
}

size_t decode_resident_lds(int k, int dtype, int cache, int head_dim, int waves) {
  size_t dyn;
  if (cache == 1)
    dyn = resident_dyn_lds_t<bf16, e4m3>(k, head_dim);
  else if (dtype == 0)
    dyn = resident_dyn_lds_t<float, float>(k, head_dim);
  else
    dyn = resident_dyn_lds_t<bf16, bf16>(k, head_dim);
  return decode_static_lds(dtype, cache, head_dim, waves) + dyn;
}

int decode_multi_per_cu(int k, int dtype, int cache, int head_dim, int waves) {
  if (!decode_multi_fits(k, dtype, cache, head_dim, waves)) return 0;
  if (cache == 1) return dtype == 1 ? multi_per_cu_t<bf16, e4m3>(k, head_dim, waves) : 0;
  if (dtype == 0) return multi_per_cu_t<float, float>(k, head_dim, waves);
  if (dtype == 1) return multi_per_cu_t<bf16, bf16>(k, head_dim, waves);
  return 0;
}

hipError_t launch_decode_multi(const DecodeArgs& a, int dtype, int cache, int head_dim, int waves, int n_steps,
                               int live0, bool resident, hipStream_t s) {
  if (!decode_multi_fits(a.k, dtype, cache, head_dim, waves)) return hipErrorInvalidValue;
  if (cache == 1) {
    if (dtype != 1) return hipErrorInvalidValue;
    return launch_multi_t<bf16, e4m3>(a, head_dim, waves, n_steps, live0, resident, s);
  }
  if (dtype == 0) return launch_multi_t<float, float>(a, head_dim, waves, n_steps, live0, resident, s);
  if (dtype == 1) return launch_multi_t<bf16, bf16>(a, head_dim, waves, n_steps, live0, resident, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int cache, int head_dim, int waves,
                         const SplitScratch* sp, hipStream_t s) {
  if (cache == 1) {
    if (dtype != 1) return hipErrorInvalidValue;
    return launch_t<bf16, e4m3>(a, head_dim, waves, sp, s);
  }
  if (dtype == 0) return launch_t<float, float>(a, head_dim, waves, sp, s);
  if (dtype == 1) return launch_t<bf16, bf16>(a, head_dim, waves, sp, s);
  return hipErrorInvalidValue;
}

}  // namespace h2o
