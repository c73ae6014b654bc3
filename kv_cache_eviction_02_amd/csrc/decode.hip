// Fused H2O decode step for gfx950: attention over the cached slots and the new
// token, accumulated-score update, eviction argmin and in-place admission, in
// one kernel launch with one workgroup per (batch, head) unit.
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
// Data movement: K and V rows are streamed once from HBM with 16-byte loads,
// a row spread over D*sizeof(T)/16 consecutive lanes (8, 12 or 16 lanes for
// bf16 d = 64, 96, 128).  Each row group keeps an online softmax (running max,
// running sum, running output), so K and V are read in the same pass; the
// groups are merged through LDS at the end.  Logits are kept in LDS (k + 1
// floats) to form the exact normalised weights for the score update.  The
// argmin is a deterministic u64 minimum over (score bits << 32 | position);
// non-negative float bit patterns order like unsigned integers, so equal
// scores send the older position out.  The ring row that may move to the
// victim's slot and the new token's row are kept in LDS from the streaming
// pass, so admission writes at most two rows without reading them again.
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

template <typename T, int D, int NW, int U>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using E = Elem<T>;
  constexpr int EPL = E::kPer16B;       // elements per lane per row
  constexpr int LPR = D / EPL;          // lanes holding one row
  constexpr int G = ceil_pow2(LPR);     // lanes per row group
  constexpr int RW = 64 / G;            // rows per wave per pass
  constexpr int NG = NW * RW;           // row groups per workgroup
  constexpr int NT = NW * 64;
  constexpr int ROWB = D * E::kBytes;
  constexpr int PF = 8;                 // scores prefetched per thread
  static_assert(LPR * EPL == D && G <= 64, "row mapping");

  __shared__ float s_o[NG][D];
  __shared__ float s_m[NG];
  __shared__ float s_l[NG];
  __shared__ uint4 s_ring[2][LPR];      // K, V of the ring slot leaving the window
  __shared__ uint4 s_self[2][LPR];      // K, V of the decoded token
  __shared__ unsigned long long s_key[NW];
  __shared__ int s_victim;
  extern __shared__ float s_logit[];    // [n_live + 1] logits, later updated scores

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int gl = lane & (G - 1);
  const int grp = wave * RW + lane / G;
  const bool act = gl < LPR;

  const int k = a.k, r = a.r, t = a.t;
  const int n_ring = a.n_ring;
  const int n_live = n_ring + a.n_heavy;
  const int n_att = n_live + 1;
  const bool full = (n_live == k);
  const int ring_slot = t % r;
  const bool ring_live = ring_slot < n_ring;

  const size_t ubase = (size_t)unit * k;
  char* Kb = (char*)a.k_slots + ubase * ROWB;
  char* Vb = (char*)a.v_slots + ubase * ROWB;
  const char* kn = (const char*)a.k_new + (size_t)unit * ROWB;
  const char* vn = (const char*)a.v_new + (size_t)unit * ROWB;
  const char* qp = (const char*)a.q + (size_t)unit * ROWB;
  float* score = a.score + ubase;
  int32_t* pos = a.pos + ubase;

  // Logical row j: live ring slots [0, n_ring), then live heavy slots, then the new token.
  auto slot_of = [&](int j) { return j < n_ring ? j : r + (j - n_ring); };
  auto is_cand = [&](int s) { return full && (s >= r || s == ring_slot); };

  if (tid == 0) s_victim = ring_slot;  // overwritten by the argmin owner when the cache is full

  float qf[EPL];
  E::unpack(act ? load16(qp + gl * 16) : make_uint4(0, 0, 0, 0), qf);

  // Scores this thread updates after the pass, and positions of eviction candidates.
  float sc_pf[PF];
  int ps_pf[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int j = tid + i * NT;
    sc_pf[i] = 0.f;
    ps_pf[i] = 0;
    if (j < n_live) {
      const int s = slot_of(j);
      sc_pf[i] = score[s];
      if (is_cand(s)) ps_pf[i] = pos[s];
    }
  }

  float m = -INFINITY, lsum = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  // Row batches of NG * U rows.  Loads are unconditional (rows past the end and
  // idle lanes re-read a valid row and are masked out afterwards) so that the
  // compiler can track outstanding loads exactly; the next batch is in flight
  // while the current one is consumed.
  constexpr int STEP = NG * U;
  auto fetch = [&](int base, uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NG + grp;
      const char* kp = kn;
      const char* vp = vn;
      if (j < n_live) {
        const size_t off = (size_t)slot_of(j) * ROWB;
        kp = Kb + off;
        vp = Vb + off;
      }
      const int c = act ? gl : 0;
      kr[u] = load16_stream(kp + c * 16);
      vr[u] = load16_stream(vp + c * 16);
    }
  };
  auto consume = [&](int base, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
    float lg[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      E::unpack(kr[u], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qf[e], kf[e], d);  // qf is 0 on idle lanes
      d = group_sum<G>(d);
      const int j = base + u * NG + grp;
      lg[u] = j < n_att ? d * a.scale_log2 : -INFINITY;
      if (j < n_att) {
        if (gl == 0) s_logit[j] = lg[u];
        if (act) {
          if (j == n_live) {
            s_self[0][gl] = kr[u];
            s_self[1][gl] = vr[u];
          } else if (ring_live && j == ring_slot) {
            s_ring[0][gl] = kr[u];
            s_ring[1][gl] = vr[u];
          }
        }
      }
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, lg[u]);
    if (mn > -INFINITY) {
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(lg[u] - mn);  // 0 for rows past the end
        float vf[EPL];
        E::unpack(vr[u], vf);
        lsum += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e]);
      }
      m = mn;
    }
  };

  uint4 ka[U], va[U], kb[U], vb[U];
  fetch(0, ka, va);
  for (int base = 0; base < n_att; base += 2 * STEP) {
    fetch(base + STEP, kb, vb);
    consume(base, ka, va);
    fetch(base + 2 * STEP, ka, va);
    consume(base + STEP, kb, vb);
  }

  // Merge the row groups: global max M, normaliser L, output.
  if (gl == 0) {
    s_m[grp] = m;
    s_l[grp] = lsum;
  }
  if (act) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_o[grp][gl * EPL + e] = o[e];
  }
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < NG; ++g) M = fmaxf(M, s_m[g]);
  float wg[NG];
  float L = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    wg[g] = fast_exp2(s_m[g] - M);
    L = fmaf(s_l[g], wg[g], L);
  }
  const float invL = 1.f / L;
  for (int c = tid; c < D; c += NT) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) acc = fmaf(s_o[g][c], wg[g], acc);
    a.out[(size_t)unit * D + c] = acc * invL;
  }
  const float p_self = fast_exp2(s_logit[n_live] - M) * invL;

  // Score update; u64 argmin over the candidates.
  unsigned long long best = ~0ull;
  int best_slot = -1;
  auto update = [&](int j, float old, int ps) {
    const int s = slot_of(j);
    const float ns = old + fast_exp2(s_logit[j] - M) * invL;
    s_logit[j] = ns;
    if (is_cand(s)) {
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
    if (j < n_live) update(j, sc_pf[i], ps_pf[i]);
  }
  for (int j = tid + PF * NT; j < n_live; j += NT) {
    const int s = slot_of(j);
    update(j, score[s], is_cand(s) ? pos[s] : 0);
  }

  unsigned long long vkey = ~0ull;
  if (full) {
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
    if (best_slot >= 0 && best == vkey) s_victim = best_slot;
  }
  __syncthreads();

  // Where the row leaving the window goes: the victim's heavy slot, or the next
  // free heavy slot while the cache is not yet full; -1 if it is dropped or
  // still inside the window.
  int dst = -1;
  if (full) {
    const int victim = s_victim;
    if (victim != ring_slot) dst = victim;
  } else if (ring_live) {
    dst = r + a.n_heavy;
  }

  auto write_score = [&](int j) {
    const int s = slot_of(j);
    if (s != ring_slot && s != dst) score[s] = s_logit[j];
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int j = tid + i * NT;
    if (j < n_live) write_score(j);
  }
  for (int j = tid + PF * NT; j < n_live; j += NT) write_score(j);

  if (tid == 0) {
    if (dst >= 0) {
      score[dst] = s_logit[ring_slot];
      pos[dst] = t - r;
    }
    score[ring_slot] = p_self;
    pos[ring_slot] = t;
    if (a.evicted) a.evicted[unit] = full ? (int32_t)(uint32_t)vkey : -1;
  }
  if (tid < LPR) {
    if (dst >= 0) {
      store16(Kb + (size_t)dst * ROWB + tid * 16, s_ring[0][tid]);
      store16(Vb + (size_t)dst * ROWB + tid * 16, s_ring[1][tid]);
    }
    store16(Kb + (size_t)ring_slot * ROWB + tid * 16, s_self[0][tid]);
    store16(Vb + (size_t)ring_slot * ROWB + tid * 16, s_self[1][tid]);
  }
}

template <typename T, int D, int NW>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t s) {
  constexpr int U = 1;  // more loads in flight per wave measured slower at opt30b and neox20b
  const int n_live = a.n_ring + a.n_heavy;
  const size_t lds = (size_t)(n_live + 1) * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<T, D, NW, U>), dim3(a.units), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, int waves, hipStream_t s) {
  switch (waves) {
    case 1: return launch_nw<T, D, 1>(a, s);
    case 2: return launch_nw<T, D, 2>(a, s);
    case 4: return launch_nw<T, D, 4>(a, s);
    case 8: return launch_nw<T, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, int head_dim, int waves, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<T, 64>(a, waves, s);
    case 96: return launch_d<T, 96>(a, waves, s);
    case 128: return launch_d<T, 128>(a, waves, s);
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

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int waves, hipStream_t s) {
  if (dtype == 0) return launch_t<float>(a, head_dim, waves, s);
  if (dtype == 1) return launch_t<bf16>(a, head_dim, waves, s);
  return hipErrorInvalidValue;
}

}  // namespace h2o
