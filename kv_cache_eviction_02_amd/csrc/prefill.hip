// H2O prefill for gfx950: accumulated attention of every prompt position and the
// initial choice of recent + heavy-hitter slots.
//
// Method (H2O summary "H2O: Heavy-Hitter Oracle for Efficient Generative
// Inference", "Algorithm / figure walkthrough" step 1 and "The mechanism",
// Heavy Hitters): the score of prompt position j is the column sum
//   c_j = sum_{i >= j} softmax_i(scale * q_i . k_j),
// the total causal attention it received from the prompt's own queries.  The
// newest r positions are kept as the protected window; of the older ones the
// h largest c_j are kept (ties keep the newer position); a prompt of at most
// k = r + h positions is kept whole.
//
// Three kernels:
//   rowstats : per query row i, lse_i = m_i + log2(sum_j exp2(s_ij - m_i)) with
//              s in the log2 domain, from S^T tiles on MFMA (attend replaces it
//              when the prompt's attention output is requested);
//   colsum   : c_j = sum_i exp2(s_ij - lse_i), recomputing the S tiles on MFMA;
//              each wavefront owns 32 columns and walks the query rows in a
//              fixed order, so the sums are deterministic without atomics;
//   select   : per unit, radix select of the h largest c_j among the older
//              positions, then the gather of the heavy K/V rows into slots
//              (quantized to E4M3 with per-row scales for an E4M3 cache); the
//              window's rows, which no score decides, are copied by rowstats
//              (or attend) while it runs.
// The moving operand of both sweeps goes through LDS in chunks of 32 rows
// shared by a block's four wavefronts, staged through registers one stage
// ahead.  In each stage a wavefront reads the next chunk's fragments from LDS,
// runs the current chunk's exponentials while they arrive, then the next
// chunk's MFMAs.  A unit's blocks run on one XCD, longest first; the last
// units of each XCD's range are interleaved so that no long block starts last.
//
// MFMA use: v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (f32).
// Lane l supplies row l % 16 of a 16-row tile; of each 64-byte piece i of the
// row it supplies the 16 bytes at 64 i + 16 (l / 16), the i-th 16-byte chunk of
// its fragment.  A and B use the same split, so every product q_c * k_c is
// formed exactly once.  In LDS, rows are ROWB + 32 bytes apart: with that
// stride and this split the 16 rows of a subtile read by one ds_read_b128 fall
// on distinct banks (measured on gfx950: no bank-conflict cycles, where the
// contiguous-quarter split at a ROWB + 16 stride spent half the LDS cycles in
// conflicts).  The
// 16x16 result lands as acc[i] = dot(moving row 4 * (l / 16) + i, fixed row l % 16).
#include <float.h>
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace h2o {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kTile = 16;

template <typename T, int D>
struct Frag {
  static constexpr int kBytes = D / 4 * Elem<T>::kBytes;  // per lane: a quarter of the row
  static constexpr int kChunks = kBytes / 16;
  static_assert(kChunks * 16 == kBytes, "quarter row must be whole 16-byte chunks");
  uint4 c[kChunks];

  // Row `row0 + lane % 16` of a [n, D] matrix, chunks 64 i + 16 (lane / 16); zero past n.
  __device__ inline void load(const char* base, int row0, int n, int lane) {
    const int row = row0 + (lane & 15);
    if (row < n) {
      const char* p = base + (size_t)row * (D * Elem<T>::kBytes) + (lane >> 4) * 16;
#pragma unroll
      for (int i = 0; i < kChunks; ++i) c[i] = load16(p + 64 * i);
    } else {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) c[i] = make_uint4(0, 0, 0, 0);
    }
  }

  // Row min(row0 + lane % 16, n - 1): an unconditional load (the compiler then
  // counts outstanding loads exactly); rows past n hold a copy of row n - 1 and
  // must be masked by the caller.
  __device__ inline void load_clamped(const char* base, int row0, int n, int lane) {
    const int row = min(row0 + (lane & 15), n - 1);
    const char* p = base + (size_t)row * (D * Elem<T>::kBytes) + (lane >> 4) * 16;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) c[i] = load16(p + 64 * i);
  }
};

// acc[i] = dot(moving row 4*(lane/16)+i, fixed row lane%16)
template <typename T, int D>
__device__ inline f32x4 tile_dot(const Frag<T, D>& mv, const Frag<T, D>& fx) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < Frag<T, D>::kChunks; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, mv.c[i]),
                                                    __builtin_bit_cast(bf16x8, fx.c[i]), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < Frag<T, D>::kChunks; ++i) {
      const uint32_t a4[4] = {mv.c[i].x, mv.c[i].y, mv.c[i].z, mv.c[i].w};
      const uint32_t b4[4] = {fx.c[i].x, fx.c[i].y, fx.c[i].z, fx.c[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a4[e]), __uint_as_float(b4[e]), acc, 0, 0, 0);
    }
  }
  return acc;
}

// Blocks of one unit are kept on one XCD (blocks are dispatched round-robin over
// the 8 XCDs), so a unit's Q and K tiles are shared through that XCD's L2.
__device__ inline int xcd_local_block(int total) {
  const int L = blockIdx.x;
  if (total % 8 != 0) return L;
  return (L % 8) * (total / 8) + L / 8;
}

// Sweep blocks: id = unit * nblk + j, where j = 0 is the unit's longest block,
// so each XCD takes its units one after another, longest block first.  The
// last kTailUnits units of each XCD's range are interleaved instead (all their
// longest blocks, then all their second longest, ...): otherwise the final
// unit's longest block starts last and runs alone at the end of the launch.
constexpr int kTailUnits = 16;
__device__ inline int sweep_block(int total, int nblk) {
  int id = xcd_local_block(total);
  const int n = total / 8;  // blocks per XCD
  if (total % 8 == 0 && n % nblk == 0) {
    const int x0 = id - id % n;
    const int i = id - x0;
    const int wu = min(kTailUnits, n / nblk);
    const int w0 = n - wu * nblk;
    if (i >= w0) {
      const int k = i - w0;
      id = x0 + w0 + (k % wu) * nblk + k / wu;
    }
  }
  return id;
}

constexpr int kWaves = 4;  // wavefronts per block, each with its own rows

// Fixed 16-row subtiles held by one wavefront (B operands): 64 rows for bf16,
// 32 for f32 (whose fragments are twice as large).
template <typename T>
constexpr int kFixed = sizeof(T) == 2 ? 4 : 2;

template <typename T>
constexpr int rows_per_wave() { return kFixed<T> * kTile; }

constexpr int ceil_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Cooperative copy of prompt rows into cache slots.  Unquantized caches move
// 16-byte chunks; an E4M3 cache gives each row an aligned group of lanes,
// 16 values per lane, which agree on the row maximum and write the codes of
// x * (448 / amax) and the row scale amax / 448.
template <typename T, typename C, int D>
struct RowCopy {
  static constexpr bool kQuant = std::is_same<C, e4m3>::value;
  static constexpr int IROWB = D * Elem<T>::kBytes;   // prompt row bytes
  static constexpr int CROWB = D * Elem<C>::kBytes;   // slot row bytes
  static constexpr int ITEMS = kQuant ? D / 16 : IROWB / 16;  // work items per row
  static constexpr int GW = kQuant ? ceil_pow2(ITEMS) : ITEMS;  // loop slots per row

  // E4M3: item c of prompt row p, loaded (K's 16 values, then V's).
  __device__ static inline void load_q(const PrefillArgs& a, int unit, int P, int p, int c, uint4 (&x)[4]) {
    const int cc = c < ITEMS ? c : 0;
    const char* Kp = (const char*)a.pk + ((size_t)unit * P + p) * IROWB + cc * 32;
    const char* Vp = (const char*)a.pv + ((size_t)unit * P + p) * IROWB + cc * 32;
    x[0] = load16(Kp);
    x[1] = load16(Kp + 16);
    x[2] = load16(Vp);
    x[3] = load16(Vp + 16);
  }
  // E4M3: the codes and row scales of a loaded item, into slot sl.  Every lane
  // of the row's group takes part (the row maximum is a group reduction).
  __device__ static inline void store_q(const PrefillArgs& a, int unit, int k, int sl, int c, const uint4 (&x)[4]) {
    const bool act = c < ITEMS;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float v[16];
      Elem<T>::unpack(x[2 * w], v);
      Elem<T>::unpack(x[2 * w + 1], v + 8);
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
      amax = group_max<GW>(act ? amax : 0.f);
      char* dst = (char*)(w ? a.v_slots : a.k_slots) + ((size_t)unit * k + sl) * CROWB;
      if (act) store16(dst + c * 16, quantize16_e4m3(v, amax));
      if (c == 0) (w ? a.v_scale : a.k_scale)[(size_t)unit * k + sl] = __fdiv_rn(amax, 448.f);
    }
  }

  // item c (0 <= c < GW) of prompt row p -> slot sl
  __device__ static inline void item(const PrefillArgs& a, int unit, int P, int k, int p, int sl, int c) {
    if constexpr (!kQuant) {
      const char* Kp = (const char*)a.pk + ((size_t)unit * P + p) * IROWB;
      const char* Vp = (const char*)a.pv + ((size_t)unit * P + p) * IROWB;
      char* Ks = (char*)a.k_slots + ((size_t)unit * k + sl) * CROWB;
      char* Vs = (char*)a.v_slots + ((size_t)unit * k + sl) * CROWB;
      store16(Ks + c * 16, load16(Kp + c * 16));
      store16(Vs + c * 16, load16(Vp + c * 16));
    } else {
      uint4 x[4];
      load_q(a, unit, P, p, c, x);
      store_q(a, unit, k, sl, c, x);
    }
  }
};

// The protected window, the newest n_ring = min(P, r) prompt positions (slot
// p % r), is kept whatever the scores are (H2O summary, "The mechanism": the
// recent window beside the heavy hitters).  The sweep over query rows (row
// statistics, or the prompt output) therefore copies its rows into their slots
// while the launch runs, a phase that leaves the memory system mostly idle,
// and the selection afterwards copies only the heavy rows.
//
// A block that copies pays about one memory latency for it: stores issued
// mid-sweep make the next tile-load wait also wait for their acknowledgement
// (vector-memory completions are counted in issue order), and a copy after the
// sweep waits for its own loads.  So the window goes to the two shortest blocks
// of each unit (blk 0 and 1), which copy it after their sweep with 8 items
// (E4M3: 4, at d = 64 2) per thread in flight.  Measured at opt30b, the row
// statistics then cost what they did without the copy, where copying in all
// eight blocks cost them 5%.  E4M3 rows are quantized one aligned lane group
// per row.
template <typename T, typename C, int D>
struct WindowCopy {
  using RC = RowCopy<T, C, D>;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlocks = 2;  // blocks of a unit that copy (blk < kBlocks)
  int first, r, i0, i1;              // window rows start at position `first`; items [i0, i1), item = row * GW + c

  __device__ inline WindowCopy(const PrefillArgs& a, int blk, int nblk) {
    const int n_ring = min(a.P, a.r);
    first = a.P - n_ring;
    r = a.r;
    const int nb = min(kBlocks, nblk);
    i0 = blk < nb ? (int)((long long)n_ring * blk / nb) * RC::GW : 0;
    i1 = blk < nb ? (int)((long long)n_ring * (blk + 1) / nb) * RC::GW : 0;
  }
  __device__ inline int pos_of(int i) const { return first + i / RC::GW; }
  __device__ inline size_t src_off(int unit, int P, int i) const {
    return ((size_t)unit * P + pos_of(i)) * RC::IROWB + (i % RC::GW) * 16;
  }
  __device__ inline size_t dst_off(int unit, int k, int i) const {
    return ((size_t)unit * k + pos_of(i) % r) * RC::CROWB + (i % RC::GW) * 16;
  }
  // This block's share, after its sweep.  Called by every thread of the block.
  __device__ inline void copy(const PrefillArgs& a, int unit) {
    const int tid = threadIdx.x;
    if constexpr (!RC::kQuant) {
      constexpr int RB = 8;  // items per thread loaded before any is stored
      for (int base = i0; base < i1; base += RB * kThreads) {
        uint4 kb[RB], vb[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const size_t off = src_off(unit, a.P, min(base + tid + u * kThreads, i1 - 1));
          kb[u] = load16((const char*)a.pk + off);
          vb[u] = load16((const char*)a.pv + off);
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int i = base + tid + u * kThreads;
          if (i < i1) {
            const size_t off = dst_off(unit, a.k, i);
            store16((char*)a.k_slots + off, kb[u]);
            store16((char*)a.v_slots + off, vb[u]);
          }
        }
      }
    } else {
      // i0 and i1 are whole rows and GW divides the block, so a row's lane
      // group is in or out together.  The loads of QB items per thread are
      // issued before any of them is quantized.
      constexpr int QB = D >= 96 ? 4 : 2;  // d = 64: 2 keeps the row statistics' occupancy
      for (int base = i0; base < i1; base += QB * kThreads) {
        uint4 x[QB][4];
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int i = min(base + tid + u * kThreads, i1 - 1);
          RC::load_q(a, unit, a.P, pos_of(i), i % RC::GW, x[u]);
        }
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int i = base + tid + u * kThreads;
          if (i < i1) RC::store_q(a, unit, a.k, pos_of(i) % r, i % RC::GW, x[u]);
        }
      }
    }
  }
};

// ---- prompt attention output --------------------------------------------------
//
// O_i = sum_{j <= i} softmax_i(s_ij) v_j for every prompt row (the full causal
// attention the prompt is processed with before any eviction), computed in the
// sweep that owns query rows, which then also writes lse_i for the column sums.
// Keys and values go through LDS in chunks of 32 rows shared by the block's four
// wavefronts; each wavefront owns 32 queries as two fixed 16-row subtiles.
//   S^T tiles: acc[i] = s(key 16*sub + 4*(l/16) + i, query l%16), as in rowstats.
//   O^T tiles: D[col][query] = sum_key V[key][col] P[query][key] on the same
//              MFMA.  Lane (g, n) passes the eight probabilities it holds for
//              query n (chunk rows 16*(e/4) + 4g + e%4, e = 0..7) as the B
//              operand; the A operand carries the same eight rows of column
//              16*dt + n.  For bf16 two ds_read_b64_tr_b16 fetch them from the
//              row-major V chunk: within each 16-lane block that instruction
//              returns element e of lane L from element L%4 of lane 4e + L/4, so
//              lane s of block g addresses row 4g + s/4, column 16*dt + 4*(s%4).
// The four lane groups holding a query share its running maximum, so the 32
// probabilities of a chunk enter one MFMA.  The maximum is raised only when a
// chunk exceeds it by more than kLazy (log2 units): unnormalised probabilities
// stay below 2^kLazy and most chunks need no rescale of the accumulators.
template <typename T, int D>
struct AttendTile {
  static constexpr int QS = 2;  // fixed query subtiles per wavefront (the output accumulators limit it)
  static constexpr int ROWS = QS * kTile;             // queries per wavefront
  static constexpr int BQ = kWaves * ROWS;            // queries per block
  static constexpr int KC = 2 * kTile;                // keys per chunk
  static constexpr int ROWB = D * Elem<T>::kBytes;
  static constexpr int KSTR = ROWB + 32;              // K rows in LDS: 16 rows of one subtile hit distinct banks
  static constexpr int VSTR = ROWB + 32;              // V rows in LDS: 8 rows x 32 bytes hit distinct banks
  static constexpr int PIECES = KC * ROWB / 16;       // 16-byte pieces of a K (or V) chunk
  static constexpr int PER_T = (PIECES + kWaves * 64 - 1) / (kWaves * 64);
  static constexpr int NDT = D / 16;                  // 16-wide output column tiles
  static constexpr int BUF = KC * (KSTR + VSTR);      // bytes of one K + V chunk
  static constexpr int NBUF = 2 * BUF <= 60 * 1024 ? 2 : 1;
};

constexpr float kLazy = 8.f;
constexpr float kRescale = 0x1p64f;  // row statistics: largest chunk sum taken without a rescale

// x, or zeros when !keep (a value select: no branch, no address select).
__device__ inline uint4 zero_unless(bool keep, uint4 x) {
  return make_uint4(keep ? x.x : 0u, keep ? x.y : 0u, keep ? x.z : 0u, keep ? x.w : 0u);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Rows row0 .. row0 + 15 of a chunk in LDS as MFMA operands (lane: row l%16, chunks 64 i + 16 (l/16)).
template <typename T, int D>
__device__ inline void load_lds_frag(Frag<T, D>& f, const char* base, int row0, int stride, int lane) {
  const char* p = base + (row0 + (lane & 15)) * stride + (lane >> 4) * 16;
#pragma unroll
  for (int i = 0; i < Frag<T, D>::kChunks; ++i) f.c[i] = *reinterpret_cast<const uint4*>(p + 64 * i);
}

template <typename T, typename C, int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void attend_kernel(
    PrefillArgs a, int stride, int nblk) {
  using AT = AttendTile<T, D>;
  constexpr int QS = AT::QS;
  constexpr int NDT = AT::NDT;
  constexpr float kLow = -1.0e30f;
  __shared__ __attribute__((aligned(16))) char smem[AT::NBUF * AT::BUF];

  const int id = sweep_block(nblk * a.units, nblk);
  const int unit = id / nblk;
  const int blk = nblk - 1 - id % nblk;  // longest rows first
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int P = a.P;
  const int qb0 = blk * AT::BQ;
  const int qw0 = qb0 + __builtin_amdgcn_readfirstlane(tid >> 6) * AT::ROWS;  // first query of this wavefront
  const int qw_last = min(qw0 + AT::ROWS, P) - 1;   // < qw0 when the wavefront has no query
  const int kend = min(P, qb0 + AT::BQ);            // keys the block needs
  const int nch = (kend + AT::KC - 1) / AT::KC;
  const char* Qb = (const char*)a.pq + (size_t)unit * P * AT::ROWB;
  const char* Kb = (const char*)a.pk + (size_t)unit * P * AT::ROWB;
  const char* Vb = (const char*)a.pv + (size_t)unit * P * AT::ROWB;
  const float sc = a.scale_log2;

  Frag<T, D> fq[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) fq[q].load(Qb, qw0 + q * kTile, P, lane);
  float m[QS], l[QS];
  f32x4 o[QS][NDT];
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    m[q] = kLow;
    l[q] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[q][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Chunk loads are unconditional (a clamped address) so the compiler tracks
  // them exactly and the next chunk stays in flight during the multiply; rows
  // past the block's keys are replaced by zeros when they are stored.
  uint4 rk[AT::PER_T], rv[AT::PER_T];
  auto fetch = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < AT::PER_T; ++u) {
      const int idx = min(tid + u * kWaves * 64, AT::PIECES - 1);
      const int key = min(ch * AT::KC + idx / (AT::ROWB / 16), kend - 1);
      const int c16 = idx % (AT::ROWB / 16);
      rk[u] = load16(Kb + (size_t)key * AT::ROWB + c16 * 16);
      rv[u] = load16(Vb + (size_t)key * AT::ROWB + c16 * 16);
    }
  };
  auto stash = [&](int ch, int b) __attribute__((always_inline)) {
    char* kl = smem + b * AT::BUF;
    char* vl = kl + AT::KC * AT::KSTR;
#pragma unroll
    for (int u = 0; u < AT::PER_T; ++u) {
      const int idx = tid + u * kWaves * 64;
      if (idx < AT::PIECES) {
        const int row = idx / (AT::ROWB / 16);
        const int c16 = idx % (AT::ROWB / 16);
        // zeros past the block's keys: only the last chunk can reach them (uniform test)
        const bool tail = (ch + 1) * AT::KC > kend;
        const bool in = !tail || ch * AT::KC + row < kend;
        *reinterpret_cast<uint4*>(kl + row * AT::KSTR + c16 * 16) = tail ? zero_unless(in, rk[u]) : rk[u];
        *reinterpret_cast<uint4*>(vl + row * AT::VSTR + c16 * 16) = tail ? zero_unless(in, rv[u]) : rv[u];
      }
    }
  };

  // One body for masked and unmasked chunks: a second copy of the value
  // product (as the row statistics use) would not fit the register budget.
  auto compute = [&](int ch, const char* kl, const char* vl) __attribute__((always_inline)) {
    const int c0 = ch * AT::KC;
    f32x4 s[2][QS];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      Frag<T, D> fk;
      load_lds_frag<T, D>(fk, kl, sub * kTile, AT::KSTR, lane);
#pragma unroll
      for (int q = 0; q < QS; ++q) s[sub][q] = tile_dot<T, D>(fk, fq[q]);
    }
    // Causal mask.  Keys past P follow every query row < P; rows past P are not
    // written, so the causal test alone suffices.  Key 16*sub + 4g + i of the
    // chunk is kept for query qi iff 16*sub + i <= qi - c0 - 4g.
    if (c0 + AT::KC - 1 > qw0) {  // uniform
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        const int t = qw0 + q * kTile + (lane & 15) - c0 - 4 * g;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[sub][q][i] = sub * kTile + i <= t ? s[sub][q][i] : -INFINITY;
      }
    }
    float alpha[QS];
    bool raise_any = false;
    f32x4 p[2][QS];
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      float mx = fmaxf(s[0][q][0], s[0][q][1]);  // a chain of 3-input maxima
      mx = fmaxf(fmaxf(mx, s[0][q][2]), s[0][q][3]);
      mx = fmaxf(fmaxf(mx, s[1][q][0]), s[1][q][1]);
      mx = fmaxf(fmaxf(mx, s[1][q][2]), s[1][q][3]);
      // one maximum for the four lane groups of a query
      mx = max_pair<false>(mx);
      mx = max_pair<true>(mx);
      const float ms = mx * sc;
      const bool raise = ms > m[q] + kLazy;
      const float mn = raise ? ms : m[q];
      alpha[q] = fast_exp2(m[q] - mn);
      raise_any |= raise;
      m[q] = mn;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[sub][q][i] = fast_exp2(fmaf(s[sub][q][i], sc, -mn));
      // pairwise sum: a short dependency chain
      const float add = ((p[0][q][0] + p[0][q][1]) + (p[0][q][2] + p[0][q][3])) +
                        ((p[1][q][0] + p[1][q][1]) + (p[1][q][2] + p[1][q][3]));
      l[q] = fmaf(l[q], alpha[q], add);
    }
    if (__any(raise_any)) {
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[q][dt] *= alpha[q];
    }
    if constexpr (sizeof(T) == 2) {
      bf16x8 pb[QS];
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[q][e] = (__bf16)p[e >> 2][q][e & 3];
      const int s16 = lane & 15;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const char* v0 = vl + (4 * g + (s16 >> 2)) * AT::VSTR + (16 * dt + 4 * (s16 & 3)) * 2;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)v0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + kTile * AT::VSTR));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int q = 0; q < QS; ++q)
          o[q][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[q], o[q][dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float va = *reinterpret_cast<const float*>(
                vl + (sub * kTile + 4 * g + i) * AT::VSTR + (16 * dt + (lane & 15)) * 4);
#pragma unroll
            for (int q = 0; q < QS; ++q)
              o[q][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, p[sub][q][i], o[q][dt], 0, 0, 0);
          }
    }
  };

  fetch(0);
  stash(0, 0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    if (ch + 1 < nch) fetch(ch + 1);
    const char* kl = smem + (ch % AT::NBUF) * AT::BUF;
    if (ch * AT::KC <= qw_last) compute(ch, kl, kl + AT::KC * AT::KSTR);  // uniform
    if (AT::NBUF == 1) __syncthreads();
    if (ch + 1 < nch) stash(ch + 1, (ch + 1) % AT::NBUF);
    __syncthreads();
  }
  WindowCopy<T, C, D>(a, blk, nblk).copy(a, unit);

  if (qw0 >= P) return;
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    float lt = l[q];
    lt = sum_pair<false>(lt);
    lt = sum_pair<true>(lt);
    const int qi = qw0 + q * kTile + (lane & 15);
    if (qi < P) {
      const float inv = 1.f / lt;
      float* orow = a.out + ((size_t)unit * P + qi) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4 v = o[q][dt] * inv;
        *reinterpret_cast<float4*>(orow + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) a.row_lse[(size_t)unit * stride + qi] = m[q] + __log2f(lt);
    }
  }
}

// Row statistics lse_i = m_i + log2(sum_{j <= i} exp2(s_ij - m_i)), software
// pipelined: a block's four wavefronts own 4 x RowTile::QS * 16 queries and
// walk the keys in chunks of 32 staged through LDS (double-buffered, shared by
// the wavefronts).  At chunk c a wavefront issues the MFMAs of chunk c + 1 and
// then runs the exponentials of chunk c from registers, so the matrix and
// vector pipes overlap inside the wavefront.  The running maximum is kept per
// lane group and raised only when a chunk's sum against it would exceed
// kRescale; the four lane groups of a query merge their (max, sum) at the end.
#ifndef H2O_ROW_QS
#define H2O_ROW_QS 2
#endif
// A kernel argument used inside a sweep's loop, read into its SGPR here.  The
// argument arrives by a scalar load, and scalar loads share the lgkm counter
// with LDS reads but complete out of order: were the load left to the loop's
// first use, the wait for it there would be lgkmcnt(0) in every stage, holding
// the exponentials until the next chunk's LDS reads had returned.
__device__ inline float pin_arg(float v) {
  asm volatile("" : "+s"(v));
  return v;
}

template <typename T, int D>
struct RowTile {
  static constexpr int QS = sizeof(T) == 2 ? H2O_ROW_QS : 2;  // fixed query subtiles per wavefront
  static constexpr int ROWS = QS * kTile;
  static constexpr int BQ = kWaves * ROWS;
  static constexpr int KC = 2 * kTile;
  static constexpr int ROWB = D * Elem<T>::kBytes;
  static constexpr int KSTR = ROWB + 32;  // 16 rows of one subtile hit distinct banks
  static constexpr int PIECES = KC * ROWB / 16;
  static constexpr int PER_T = (PIECES + kWaves * 64 - 1) / (kWaves * 64);
  static constexpr int BUF = KC * KSTR;
};

template <typename T, typename C, int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void rowstats_kernel(
    PrefillArgs a, int stride, int nblk) {
  using RT = RowTile<T, D>;
  constexpr int QS = RT::QS;
  constexpr float kLow = -1.0e30f;
  __shared__ __attribute__((aligned(16))) char smem[2 * RT::BUF];

  const int id = sweep_block(nblk * a.units, nblk);
  const int unit = id / nblk;
  const int blk = nblk - 1 - id % nblk;  // longest rows first
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int P = a.P;
  const int qb0 = blk * RT::BQ;
  const int qw0 = qb0 + __builtin_amdgcn_readfirstlane(tid >> 6) * RT::ROWS;
  const int qw_last = min(qw0 + RT::ROWS, P) - 1;  // < qw0 when the wavefront has no query
  const int kend = min(P, qb0 + RT::BQ);
  const int nch = (kend + RT::KC - 1) / RT::KC;
  const char* Qb = (const char*)a.pq + (size_t)unit * P * RT::ROWB;
  const char* Kb = (const char*)a.pk + (size_t)unit * P * RT::ROWB;
  const float sc = pin_arg(a.scale_log2);

  Frag<T, D> fq[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) fq[q].load_clamped(Qb, qw0 + q * kTile, P, lane);  // rows past P: not written
  float m[QS], l[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    m[q] = kLow;
    l[q] = 0.f;
  }

  uint4 rk[RT::PER_T];
  // A chunk wholly below kend is read at a per-thread 32-bit offset from the
  // chunk's (uniform) base; only the block's last chunk clamps its rows.
  uint32_t thr_off[RT::PER_T];
#pragma unroll
  for (int u = 0; u < RT::PER_T; ++u) {
    const int idx = min(tid + u * kWaves * 64, RT::PIECES - 1);
    thr_off[u] = (idx / (RT::ROWB / 16)) * RT::ROWB + (idx % (RT::ROWB / 16)) * 16;
  }
  // Chunks past the block's keys clamp their rows, so any ch is a valid fetch.
  auto fetch = [&](int ch, uint4 (&r)[RT::PER_T]) __attribute__((always_inline)) {
    if ((ch + 1) * RT::KC <= kend) {  // uniform
      const char* cb = Kb + (size_t)ch * RT::KC * RT::ROWB;
#pragma unroll
      for (int u = 0; u < RT::PER_T; ++u) r[u] = load16(cb + thr_off[u]);
    } else {
#pragma unroll
      for (int u = 0; u < RT::PER_T; ++u) {
        const int idx = min(tid + u * kWaves * 64, RT::PIECES - 1);
        const int key = min(ch * RT::KC + idx / (RT::ROWB / 16), kend - 1);
        r[u] = load16(Kb + (size_t)key * RT::ROWB + (idx % (RT::ROWB / 16)) * 16);
      }
    }
  };
  auto stash = [&](int b, const uint4 (&r)[RT::PER_T]) __attribute__((always_inline)) {
    char* kl = smem + b * RT::BUF;
#pragma unroll
    for (int u = 0; u < RT::PER_T; ++u) {
      const int idx = tid + u * kWaves * 64;
      if (RT::PIECES % (kWaves * 64) == 0 || idx < RT::PIECES)  // no branch when the block covers the chunk evenly
        *reinterpret_cast<uint4*>(kl + (idx / (RT::ROWB / 16)) * RT::KSTR + (idx % (RT::ROWB / 16)) * 16) = r[u];
    }
  };
  // Keys past kend hold copies of row kend - 1: they follow every query of the
  // block that is < P, so the causal mask removes them.
  auto read = [&](int ch, Frag<T, D> (&fk)[2]) __attribute__((always_inline)) {
    const char* kl = smem + (ch & 1) * RT::BUF;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) load_lds_frag<T, D>(fk[sub], kl, sub * kTile, RT::KSTR, lane);
  };
  auto mult = [&](const Frag<T, D> (&fk)[2], f32x4 (&s)[2][QS]) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int q = 0; q < QS; ++q) s[sub][q] = tile_dot<T, D>(fk[sub], fq[q]);
  };
  // The only chunk that needs the causal mask is the wavefront's diagonal one
  // (c0 = qw0): key 16*sub + 4g + i of it is kept for query qw0 + 16q + l%16 iff
  // 16*sub + i <= 16q + l%16 - 4g.  Its 0 / -inf terms are set once.
  float diag[QS][2][4];
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    const int t = q * kTile + (lane & 15) - 4 * g;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) diag[q][sub][i] = sub * kTile + i <= t ? 0.f : -INFINITY;
  }
  auto soft = [&](auto mask_tag, auto first_tag, int ch, f32x4 (&s)[2][QS]) __attribute__((always_inline)) {
    if constexpr (decltype(mask_tag)::value) {
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[sub][q][i] += diag[q][sub][i];
    }
    if constexpr (decltype(first_tag)::value) {
      // The wavefront's first chunk (chunk 0): m[q] is still kLow, so every
      // lane with a kept term would take the retake below.  Its maximum is
      // taken first instead (kLow for a lane whose terms are all masked),
      // which is the maximum the retake would set: the same bits, one pass of
      // exponentials, no rescale (every term is at most 1).
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        float mx = fmaxf(s[0][q][0], s[0][q][1]);
        mx = fmaxf(fmaxf(mx, s[0][q][2]), s[0][q][3]);
        mx = fmaxf(fmaxf(mx, s[1][q][0]), s[1][q][1]);
        mx = fmaxf(fmaxf(mx, s[1][q][2]), s[1][q][3]);
        m[q] = fmaxf(m[q], mx * sc);
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fmaf(s[i >> 2][q][i & 3], sc, -m[q]));
        l[q] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
      return;
    }
    // Exponentials against the running maximum m[q] without first taking the
    // chunk's maximum.  A lane whose chunk sum exceeds 2^64 (or is infinite:
    // a lane whose first chunk was all masked still has m[q] = kLow) raises
    // m[q] to the chunk's maximum and takes the chunk again: rare, and a
    // uniform branch.  Every
    // term then stays below 2^64 and one term of the sum is at least 1 (the one
    // that set m[q]), so the float sum keeps its relative precision, and no
    // sum over a row overflows.
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fmaf(s[i >> 2][q][i & 3], sc, -m[q]));
      float add = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      const bool big = !(add <= kRescale);
      if (__builtin_amdgcn_ballot_w64(big)) {  // uniform
        float mx = fmaxf(s[0][q][0], s[0][q][1]);
        mx = fmaxf(fmaxf(mx, s[0][q][2]), s[0][q][3]);
        mx = fmaxf(fmaxf(mx, s[1][q][0]), s[1][q][1]);
        mx = fmaxf(fmaxf(mx, s[1][q][2]), s[1][q][3]);
        const float mn = big ? fmaxf(m[q], mx * sc) : m[q];
        const float alpha = fast_exp2(m[q] - mn);
        m[q] = mn;
        if (big) {
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fmaf(s[i >> 2][q][i & 3], sc, -mn));
          add = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        }
        l[q] = fmaf(l[q], alpha, add);
      } else {
        l[q] += add;
      }
    }
  };
  auto active = [&](int ch) { return ch < nch && ch * RT::KC <= qw_last; };  // uniform
  // One pipeline stage: the LDS reads of chunk ch + 1 go out first, the
  // exponentials of chunk ch (S tiles from the stage before) cover their
  // latency, and the MFMAs of chunk ch + 1 then overwrite the same S registers;
  // their results are not needed before the next stage.
  auto stage = [&](auto first_tag, int ch, f32x4 (&s)[2][QS]) __attribute__((always_inline)) {
    const bool diag = ch * RT::KC + RT::KC - 1 > qw0;
    const bool next = active(ch + 1);
    if (ch + 2 < nch) fetch(ch + 2, rk);
    Frag<T, D> fk[2];
    if (next) read(ch + 1, fk);
    if (active(ch)) {
      if (diag)
        soft(std::true_type{}, first_tag, ch, s);
      else
        soft(std::false_type{}, first_tag, ch, s);
    }
    if (next) mult(fk, s);
    if (ch + 2 < nch) stash(ch & 1, rk);  // chunk ch + 2 replaces chunk ch, read one stage ago
    __syncthreads();
  };

  f32x4 s[2][QS];
  {
    // Both first chunks' loads are in flight before the first wait for either.
    // Buffer 1 is written even for a single chunk (it is then never read): a
    // conditional store would let the compiler sink chunk 1's loads behind the
    // wait for chunk 0.
    uint4 rk1[RT::PER_T];
    fetch(0, rk);
    fetch(1, rk1);
    stash(0, rk);
    stash(1, rk1);
  }
  __syncthreads();
  if (active(0)) {
    Frag<T, D> fk[2];
    read(0, fk);
    mult(fk, s);
  }
  __syncthreads();  // every wavefront has read chunk 0 before chunk 2 replaces it
  stage(std::true_type{}, 0, s);  // chunk 0 is the first chunk of every wavefront with queries
  for (int ch = 1; ch < nch; ++ch) stage(std::false_type{}, ch, s);
  WindowCopy<T, C, D>(a, blk, nblk).copy(a, unit);

  if (qw0 >= P) return;
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    float lt = l[q];
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {  // merge the lane groups' (max, sum)
      const float mo = __shfl_xor(m[q], off, 64);
      const float lo = __shfl_xor(lt, off, 64);
      const float mn = fmaxf(m[q], mo);
      lt = lt * fast_exp2(m[q] - mn) + lo * fast_exp2(mo - mn);
      m[q] = mn;
    }
    const int qi = qw0 + q * kTile + (lane & 15);
    if (g == 0 && qi < P) a.row_lse[(size_t)unit * stride + qi] = m[q] + __log2f(lt);
  }
}

// Column sums c_j = sum_{i >= j} exp2(s_ij - lse_i).  A block's four
// wavefronts own 4 x ColTile::QS * 16 consecutive keys (fixed B operands) and
// walk the query rows from the block's first key to the end of the prompt in
// chunks of 32, staged with their lse values through LDS (double-buffered,
// shared by the wavefronts).  Software pipelined like the row statistics: at
// chunk c a wavefront issues the MFMAs of chunk c + 1 (and reads its lse into
// registers), then runs the exponentials of chunk c.  Every lane accumulates
// its columns in a fixed order, so the sums are deterministic.  With
// last_row_only (naive per-step Top-K) only the last prompt row contributes:
// c_j = exp2(s_{P-1,j} - lse_{P-1}).
#ifndef H2O_COL_QS
#define H2O_COL_QS 2
#endif
template <typename T, int D>
struct ColTile {
  static constexpr int QS = sizeof(T) == 2 ? H2O_COL_QS : 2;  // fixed key subtiles per wavefront
  static constexpr int ROWS = QS * kTile;            // keys per wavefront
  static constexpr int BK = kWaves * ROWS;           // keys per block
  static constexpr int QC = 2 * kTile;               // query rows per chunk
  static constexpr int ROWB = D * Elem<T>::kBytes;
  static constexpr int QSTR = ROWB + 32;             // 16 rows of one subtile hit distinct banks
  static constexpr int PIECES = QC * ROWB / 16;
  static constexpr int PER_T = (PIECES + kWaves * 64 - 1) / (kWaves * 64);
  static constexpr int BUF = QC * QSTR + QC * 4;     // query rows + their lse
};

template <typename T, int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void colsum_kernel(
    PrefillArgs a, int stride, int nblk) {
  using CT = ColTile<T, D>;
  constexpr int QS = CT::QS;
  __shared__ __attribute__((aligned(16))) char smem[2 * CT::BUF];

  const int id = sweep_block(nblk * a.units, nblk);
  const int unit = id / nblk;
  const int blk = id % nblk;  // first columns have the most rows
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g4 = (lane >> 4) * 4;
  const int P = a.P;
  const int jb0 = blk * CT::BK;
  const int j0 = jb0 + __builtin_amdgcn_readfirstlane(tid >> 6) * CT::ROWS;  // first key of this wavefront
  const char* Qb = (const char*)a.pq + (size_t)unit * P * CT::ROWB;
  const char* Kb = (const char*)a.pk + (size_t)unit * P * CT::ROWB;
  const float* lse = a.row_lse + (size_t)unit * stride;
  const float sc = pin_arg(a.scale_log2);
  const bool last_only = a.last_row_only != 0;
  const int q_lo = last_only ? P - 1 : 0;              // first query row that counts
  const int ch0 = (last_only ? P - 1 : jb0) / CT::QC;  // first chunk the block needs
  const int nch = (P + CT::QC - 1) / CT::QC;
  const int w_last = min(j0 + CT::ROWS, P) - 1;       // last key of this wavefront (< j0: none)

  Frag<T, D> fk[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) fk[q].load_clamped(Kb, j0 + q * kTile, P, lane);  // keys past P: not written
  float cs[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) cs[q] = 0.f;

  // Unconditional chunk loads (row clamped to P - 1); rows past P are masked.
  uint4 rq[CT::PER_T];
  float rl = 0.f;
  // A chunk wholly inside the prompt is read at a per-thread 32-bit offset from
  // the chunk's (uniform) base; only the last chunk clamps its rows.
  uint32_t thr_off[CT::PER_T];
#pragma unroll
  for (int u = 0; u < CT::PER_T; ++u) {
    const int idx = min(tid + u * kWaves * 64, CT::PIECES - 1);
    thr_off[u] = (idx / (CT::ROWB / 16)) * CT::ROWB + (idx % (CT::ROWB / 16)) * 16;
  }
  // Chunks past the prompt clamp their rows, so any ch is a valid fetch.
  auto fetch = [&](int ch, uint4 (&r)[CT::PER_T], float& l) __attribute__((always_inline)) {
    if ((ch + 1) * CT::QC <= P) {  // uniform
      const char* cb = Qb + (size_t)ch * CT::QC * CT::ROWB;
#pragma unroll
      for (int u = 0; u < CT::PER_T; ++u) r[u] = load16(cb + thr_off[u]);
      if (tid < CT::QC) l = lse[ch * CT::QC + tid];
    } else {
#pragma unroll
      for (int u = 0; u < CT::PER_T; ++u) {
        const int idx = min(tid + u * kWaves * 64, CT::PIECES - 1);
        const int row = min(ch * CT::QC + idx / (CT::ROWB / 16), P - 1);
        r[u] = load16(Qb + (size_t)row * CT::ROWB + (idx % (CT::ROWB / 16)) * 16);
      }
      if (tid < CT::QC) l = lse[min(ch * CT::QC + tid, P - 1)];
    }
  };
  // Chunk c's rows and lse values go to buffer (c - ch0) & 1.
  auto stash = [&](int b, const uint4 (&r)[CT::PER_T], float l) __attribute__((always_inline)) {
    char* ql = smem + b * CT::BUF;
#pragma unroll
    for (int u = 0; u < CT::PER_T; ++u) {
      const int idx = tid + u * kWaves * 64;
      if (CT::PIECES % (kWaves * 64) == 0 || idx < CT::PIECES)  // no branch when the block covers the chunk evenly
        *reinterpret_cast<uint4*>(ql + (idx / (CT::ROWB / 16)) * CT::QSTR + (idx % (CT::ROWB / 16)) * 16) =
            r[u];
    }
    if (tid < CT::QC) reinterpret_cast<float*>(ql + CT::QC * CT::QSTR)[tid] = l;
  };
  // A chunk's query fragments and lse values, into registers (the buffer is
  // refilled one stage later), then its S tiles (acc[i]: query 4g + i of the
  // subtile, key lane % 16).
  auto read = [&](int ch, Frag<T, D> (&fq)[2]) __attribute__((always_inline)) {
    const char* ql = smem + ((ch - ch0) & 1) * CT::BUF;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) load_lds_frag<T, D>(fq[sub], ql, sub * kTile, CT::QSTR, lane);
  };
  auto read_lse = [&](int ch, float4 (&lq)[2]) __attribute__((always_inline)) {
    const float* ll = reinterpret_cast<const float*>(smem + ((ch - ch0) & 1) * CT::BUF + CT::QC * CT::QSTR);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) lq[sub] = *reinterpret_cast<const float4*>(ll + sub * kTile + g4);
  };
  auto mult = [&](const Frag<T, D> (&fq)[2], f32x4 (&s)[2][QS]) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int q = 0; q < QS; ++q) s[sub][q] = tile_dot<T, D>(fq[sub], fk[q]);
  };
  // The wavefront's diagonal query chunk (c0 = j0) inside the prompt needs
  // only the causal mask: query c0 + 16*sub + 4g + i counts for key
  // j0 + 16q + l%16 iff i >= 16q + l%16 - 16*sub - 4g.  The last chunk of a
  // ragged prompt and the last-row-only mode take the general test.
  auto soft = [&](auto edge_tag, int ch, const f32x4 (&s)[2][QS], const float4 (&lq)[2])
                  __attribute__((always_inline)) {
    constexpr int edge = decltype(edge_tag)::value;  // 0 interior, 1 diagonal, 2 general
    const int c0 = ch * CT::QC;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const float lv[4] = {lq[sub].x, lq[sub].y, lq[sub].z, lq[sub].w};
#pragma unroll
      for (int q = 0; q < QS; ++q) {
        float e[4];
        if constexpr (edge == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) e[i] = fast_exp2(fmaf(s[sub][q][i], sc, -lv[i]));
        } else if constexpr (edge == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool keep = i >= q * kTile + (lane & 15) - sub * kTile - g4;
            e[i] = fast_exp2(keep ? fmaf(s[sub][q][i], sc, -lv[i]) : -INFINITY);
          }
        } else {
          // query row base + i counts iff lo <= i < hi (causal, inside the prompt,
          // and the last row only for the naive policy); masked terms get the
          // argument -inf (exp2 gives exactly 0), so the exponential is not
          // turned into a per-lane branch
          const int base = c0 + sub * kTile + g4;
          const int lo = max(j0 + q * kTile + (lane & 15), q_lo) - base;
          const int hi = P - base;
#pragma unroll
          for (int i = 0; i < 4; ++i) e[i] = fast_exp2(i >= lo && i < hi ? fmaf(s[sub][q][i], sc, -lv[i]) : -INFINITY);
        }
        cs[q] += (e[0] + e[1]) + (e[2] + e[3]);  // pairwise: a short dependency chain
      }
    }
  };
  // uniform: the wavefront has keys and the chunk has a query at or after its first key
  auto active = [&](int ch) { return ch < nch && w_last >= j0 && (ch + 1) * CT::QC - 1 >= j0; };
  // One pipeline stage, ordered as in the row statistics: the fragments of
  // chunk ch + 1 are read from LDS, the exponentials of chunk ch (its lse
  // values read at the end of the stage before) follow, then the MFMAs of
  // chunk ch + 1 into the same S registers, and last the lse values of chunk
  // ch + 1 into the registers the exponentials have just released.  The LDS
  // reads are unconditional (the buffers always hold some chunk): with one path
  // through them the exponentials wait for the lse values alone, not for the
  // fragment reads behind them.
  auto stage = [&](int ch, f32x4 (&s)[2][QS], float4 (&lq)[2]) __attribute__((always_inline)) {
    const int c0 = ch * CT::QC;
    const bool cur = active(ch), next = active(ch + 1);
    if (ch + 2 < nch) fetch(ch + 2, rq, rl);
    Frag<T, D> fq[2];
    read(ch + 1, fq);
    if (cur) {
      if (last_only || c0 + CT::QC > P)
        soft(std::integral_constant<int, 2>{}, ch, s, lq);
      else if (c0 < j0 + CT::ROWS - 1)
        soft(std::integral_constant<int, 1>{}, ch, s, lq);
      else
        soft(std::integral_constant<int, 0>{}, ch, s, lq);
    }
    if (next) mult(fq, s);
    read_lse(ch + 1, lq);
    if (ch + 2 < nch) stash((ch - ch0) & 1, rq, rl);  // chunk ch + 2 replaces chunk ch, read one stage ago
    __syncthreads();
  };

  f32x4 s[2][QS];
  float4 lq[2];
  {
    // Both first chunks' loads are in flight before the first wait for either
    // (buffer 1 is written even when it is never read, as in the row statistics).
    uint4 rq1[CT::PER_T];
    float rl1 = 0.f;
    fetch(ch0, rq, rl);
    fetch(ch0 + 1, rq1, rl1);
    stash(0, rq, rl);
    stash(1, rq1, rl1);
  }
  __syncthreads();
  if (active(ch0)) {
    Frag<T, D> fq[2];
    read(ch0, fq);
    mult(fq, s);
  }
  read_lse(ch0, lq);
  __syncthreads();  // every wavefront has read the first chunk before the third replaces it
  for (int ch = ch0; ch < nch; ++ch) stage(ch, s, lq);
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    float c = cs[q];
    c += __shfl_xor(c, 16, 64);
    c += __shfl_xor(c, 32, 64);
    const int kj = j0 + q * kTile + lane;
    if (lane < 16 && kj < P) a.colsum[(size_t)unit * stride + kj] = c;
  }
}

constexpr int kSelThreads = 256;

// Exclusive prefix sum over the block; returns the block total in *total.
__device__ inline int block_exclusive_scan(int v, int* buf, int* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  *total = buf[kSelThreads - 1];
  __syncthreads();
  return incl - v;
}

template <typename T, typename C, int D>
__global__ __launch_bounds__(kSelThreads) void select_gather_kernel(PrefillArgs a, int stride) {
  using RC = RowCopy<T, C, D>;
  constexpr int GW = RC::GW;
  __shared__ int hist[256];
  __shared__ int buf[kSelThreads];
  __shared__ int s_digit, s_need;

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = a.P, r = a.r, h = a.h, k = a.k;
  const float* c = a.colsum + (size_t)unit * stride;
  const int n_ring = P < r ? P : r;
  const int n_pool = P - n_ring;          // positions older than the window
  const bool keep_all = n_pool <= h;
  const int n_sel = keep_all ? n_pool : h;

  float* score = a.score + (size_t)unit * k;
  int32_t* pos = a.pos + (size_t)unit * k;

  // Radix select (4 x 8 bits) of the h-th largest score bit pattern among the
  // pool; scores are >= 0 so their bits order like the values.  Each pass
  // histograms one byte among the patterns matching the prefix so far; a scan
  // over the bins from the top finds the bin holding the need-th largest.
  uint32_t thr = 0;
  int need = 0;
  if (!keep_all && h > 0) {
    uint32_t prefix = 0, mask = 0;
    need = h;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < n_pool; j += kSelThreads) {
        const uint32_t b = __float_as_uint(c[j]);
        if ((b & mask) == prefix) atomicAdd(&hist[(b >> shift) & 255], 1);
      }
      __syncthreads();
      // thread t looks at bin 255 - t: count above it (exclusive) and with it
      const int cnt = hist[255 - tid];
      int tot;
      const int above = block_exclusive_scan(cnt, buf, &tot);
      if (above < need && above + cnt >= need) {  // exactly one thread
        s_digit = 255 - tid;
        s_need = need - above;
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= 255u << shift;
      need = s_need;
      __syncthreads();
    }
    thr = prefix;
  }

  // Walk the pool from the newest position down: an equal-to-threshold score is
  // taken while fewer than `need` newer equal ones were; selected positions get
  // heavy slots in ascending position order.
  int eq_seen = 0, sel_seen = 0;
  for (int hi = n_pool; hi > 0; hi -= kSelThreads) {
    const int p = hi - 1 - tid;
    bool eq = false, gt = false;
    if (p >= 0 && !keep_all && h > 0) {
      const uint32_t b = __float_as_uint(c[p]);
      eq = b == thr;
      gt = b > thr;
    }
    int eq_total, sel_total;
    const int eq_rank = eq_seen + block_exclusive_scan(eq ? 1 : 0, buf, &eq_total);
    const bool sel = p >= 0 && (keep_all || gt || (eq && eq_rank < need));
    const int sel_rank = sel_seen + block_exclusive_scan(sel ? 1 : 0, buf, &sel_total);
    eq_seen += eq_total;
    sel_seen += sel_total;
    if (sel) {
      const int slot = r + (n_sel - 1 - sel_rank);
      score[slot] = c[p];
      pos[slot] = p;
    }
  }

  // Protected window: the newest n_ring prompt positions, slot = position % r.
  for (int i = tid; i < n_ring; i += kSelThreads) {
    const int p = P - n_ring + i;
    score[p % r] = c[p];
    pos[p % r] = p;
  }
  // Unused slots.
  for (int s = tid; s < k; s += kSelThreads) {
    const bool used = s < r ? s < n_ring : s < r + n_sel;
    if (!used) {
      score[s] = 0.f;
      pos[s] = -1;
    }
  }
  __syncthreads();  // the positions just written are read back below

  // Row copies of the heavy slots (the sweep over query rows has copied the
  // window's), GW consecutive lanes per row, each slot's source position read
  // back from pos.  For an unquantized cache every thread first issues the
  // loads of up to kBatch items, then their stores, so many rows are in flight
  // at once.
  const int n_items = n_sel * GW;
  auto slot_of_row = [&](int row) { return r + row; };
  if constexpr (!RC::kQuant) {
    constexpr int kBatch = 4;
    constexpr int IROWB = RC::IROWB;
    const char* __restrict__ Kb = (const char*)a.pk + (size_t)unit * P * IROWB;
    const char* __restrict__ Vb = (const char*)a.pv + (size_t)unit * P * IROWB;
    char* __restrict__ Ks = (char*)a.k_slots + (size_t)unit * k * RC::CROWB;
    char* __restrict__ Vs = (char*)a.v_slots + (size_t)unit * k * RC::CROWB;
    for (int base = 0; base < n_items; base += kSelThreads * kBatch) {
      uint4 kx[kBatch], vx[kBatch];
      int dst[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int idx = min(base + u * kSelThreads + tid, n_items - 1);  // clamped: loads stay in range
        const int sl = slot_of_row(idx / GW);
        const int cc = idx % GW;
        const size_t src = (size_t)pos[sl] * IROWB + cc * 16;
        kx[u] = load16(Kb + src);
        vx[u] = load16(Vb + src);
        dst[u] = sl * RC::CROWB + cc * 16;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (base + u * kSelThreads + tid < n_items) {
          store16(Ks + dst[u], kx[u]);
          store16(Vs + dst[u], vx[u]);
        }
      }
    }
  } else {
    for (int idx = tid; idx < ((n_items + kSelThreads - 1) / kSelThreads) * kSelThreads; idx += kSelThreads) {
      // whole GW-lane groups are in or out together (GW divides kSelThreads)
      if (idx < n_items) {
        const int sl = slot_of_row(idx / GW);
        RC::item(a, unit, P, k, pos[sl], sl, idx % GW);
      }
    }
  }
}

template <typename T, typename C, int D>
hipError_t launch_prefill_td(const PrefillArgs& a, int stride, hipStream_t s) {
  const dim3 block(kWaves * 64);
  if (a.out) {
    constexpr int bq = AttendTile<T, D>::BQ;
    const int nb = (a.P + bq - 1) / bq;
    hipLaunchKernelGGL((attend_kernel<T, C, D>), dim3((unsigned)(nb * a.units)), block, 0, s, a, stride, nb);
  } else {
    constexpr int bq = RowTile<T, D>::BQ;
    const int nb = (a.P + bq - 1) / bq;
    hipLaunchKernelGGL((rowstats_kernel<T, C, D>), dim3((unsigned)(nb * a.units)), block, 0, s, a, stride, nb);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int bk = ColTile<T, D>::BK;
  const int nbk = (a.P + bk - 1) / bk;
  hipLaunchKernelGGL((colsum_kernel<T, D>), dim3((unsigned)(nbk * a.units)), block, 0, s, a, stride, nbk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((select_gather_kernel<T, C, D>), dim3(a.units), dim3(kSelThreads), 0, s, a, stride);
  return hipGetLastError();
}

template <typename T, typename C>
hipError_t launch_prefill_t(const PrefillArgs& a, int head_dim, int stride, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_prefill_td<T, C, 64>(a, stride, s);
    case 96: return launch_prefill_td<T, C, 96>(a, stride, s);
    case 128: return launch_prefill_td<T, C, 128>(a, stride, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int cache, int head_dim, hipStream_t s) {
  const int stride = a.stride;
  if (cache == 1) {
    if (dtype != 1) return hipErrorInvalidValue;
    return launch_prefill_t<bf16, e4m3>(a, head_dim, stride, s);
  }
  if (dtype == 0) return launch_prefill_t<float, float>(a, head_dim, stride, s);
  if (dtype == 1) return launch_prefill_t<bf16, bf16>(a, head_dim, stride, s);
  return hipErrorInvalidValue;
}

}  // namespace h2o
