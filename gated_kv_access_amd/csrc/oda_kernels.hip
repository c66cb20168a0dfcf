// oda_kernels.hip -- gfx950 (CDNA4) kernels of the On-Demand Attention decode
// step and their launchers.
//
// Method: picx.dev summary of "On-Demand Attention", section "Local-First
// Decoding" (access sets S^L_t, S^F_t; Local pass; gate q_t > theta) and
// section "Efficient Execution" (ring KV workspace, fused cross-layer commits,
// device-side conditional Full pass).
//
// Attention is split-K flash decoding, one kernel per layer pass.  A workgroup
// of eight wave64s owns one (split, KV head, request) and streams its rows of
// K and V with 16-byte loads: every lane holds four 16-byte chunks of a row, so
// a 256-byte row (bf16, d = 128) is spread over 4 lanes and one wave covers 16
// rows per pass (FP8 E4M3 rows: two chunks per lane, two passes per tile).
// All query heads of a GQA group use each loaded row.  Scores are reduced
// across the lanes of a row with DPP and kept in the log2 domain against a
// per-lane reference maximum; the current token (position t, which the caches
// do not hold yet) is one more row, read from k_cur / v_cur by the last split.
// Ring (Local) passes use a wider geometry: one 16-byte chunk per lane and row.
// GQA groups of 4 and 8 with bf16 or FP8 K/V compute both products on MFMA
// (S^T = K Q^T, then O^T += V^T P^T with V transposed through LDS).
// Long paged passes end with a pool of tiles that the splits of a (request,
// KV head) take one at a time.  Each workgroup leaves one (o, m, l) partial per
// query head, and one workgroup of each (request, KV head) merges them into the
// output: in a launch that fits the chip at once, the highest split, reading
// the other partial slots until none is empty; otherwise the last workgroup to
// take a ticket from a counter in the workspace.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "oda_internal.h"

namespace oda {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

// Phase stamps of the profiling build (compiled with ODA_PHASE_STAMPS into
// liboda_phases.so, include/oda_phases.h; the product library has none):
// thread 0 of every attention workgroup records the chip's 100 MHz real-time
// counter at eight points of its work -- entry, request state known, first
// tile reduced, static rows done, tail pool done, fold barrier passed, partial
// stored, merge done -- and the XCD it ran on.  Slots are indexed by the
// workgroup's linear id; a launch overwrites what an earlier one left.
constexpr int kPhaseGroups = 65536;
constexpr int kPhases = 8;
#ifdef ODA_PHASE_STAMPS
__device__ unsigned long long g_phase_stamps[kPhaseGroups * kPhases];
__device__ unsigned g_phase_xcc[kPhaseGroups];
__device__ __forceinline__ int phase_slot() {
  return (int)((((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) % kPhaseGroups);
}
#define ODA_PHASE(k)                                                                    \
  do {                                                                                  \
    if (threadIdx.x == 0) g_phase_stamps[phase_slot() * kPhases + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
// A stamp taken once this wave's stores have completed.
#define ODA_PHASE_STORED(k)                          \
  do {                                               \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); \
    ODA_PHASE(k);                                    \
  } while (0)
#define ODA_PHASE_XCC()                                                            \
  do {                                                                             \
    if (threadIdx.x == 0) {                                                        \
      unsigned x;                                                                  \
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));             \
      g_phase_xcc[phase_slot()] = x & 15u;                                          \
    }                                                                              \
  } while (0)
#else
#define ODA_PHASE(k) ((void)0)
#define ODA_PHASE_STORED(k) ((void)0)
#define ODA_PHASE_XCC() ((void)0)
#endif

// ----------------------------------------------------------------------------
// lane exchange

template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
  const int x = __float_as_int(v);
  // DPP forms read a valid lane everywhere, so bound_ctrl changes nothing but
  // lets the compiler fold the move into the consuming add.
  if constexpr (MASK == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  } else if constexpr (MASK == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  } else if constexpr (MASK < 32) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x1F | (MASK << 10)));      // xor within 32
  } else {
    return __shfl_xor(v, MASK, 64);
  }
}

template <int FIRST, int LAST>
__device__ __forceinline__ float sum_over(float v) {
  if constexpr (FIRST > LAST) {
    return v;
  } else {
    v += xor_lane<FIRST>(v);
    return sum_over<FIRST * 2, LAST>(v);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate right by N lanes inside each row of 16 lanes (DPP, a VALU operand
// modifier: no LDS traffic and no wait).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, true));
}

// Sum over the LPR consecutive lanes that hold one K/V row (LPR = 2..16,
// aligned groups), left in every lane of the group: quad permutations, then
// the half-row and row mirrors (DPP, no LDS).
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += xor_lane<1>(v);
  if constexpr (LPR >= 4) v += xor_lane<2>(v);
  if constexpr (LPR >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (LPR >= 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));  // row_mirror
  return v;
}

// Sum / max over the lanes of a 16-lane row that are congruent modulo STEP
// (the row groups when a K/V row spans STEP lanes).
template <int STEP>
__device__ __forceinline__ float row_group_sum(float v) {
  if constexpr (STEP <= 8) v += row_ror<8>(v);
  if constexpr (STEP <= 4) v += row_ror<4>(v);
  if constexpr (STEP <= 2) v += row_ror<2>(v);
  if constexpr (STEP <= 1) v += row_ror<1>(v);
  return v;
}
template <int STEP>
__device__ __forceinline__ float row_group_max(float v) {
  if constexpr (STEP <= 8) v = fmaxf(v, row_ror<8>(v));
  if constexpr (STEP <= 4) v = fmaxf(v, row_ror<4>(v));
  if constexpr (STEP <= 2) v = fmaxf(v, row_ror<2>(v));
  if constexpr (STEP <= 1) v = fmaxf(v, row_ror<1>(v));
  return v;
}

// Max / sum over the 64 lanes of a wave, in every lane: DPP inside each
// 16-lane row, then the four row results read as scalars (no LDS-crossbar
// exchange on the way).
__device__ __forceinline__ float wave_max(float v) {
  const int r = __float_as_int(row_group_max<1>(v));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(r, 0)), __int_as_float(__builtin_amdgcn_readlane(r, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(r, 32)), __int_as_float(__builtin_amdgcn_readlane(r, 48))));
}
__device__ __forceinline__ float wave_sum(float v) {
  const int r = __float_as_int(row_group_sum<1>(v));
  return (__int_as_float(__builtin_amdgcn_readlane(r, 0)) + __int_as_float(__builtin_amdgcn_readlane(r, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(r, 32)) + __int_as_float(__builtin_amdgcn_readlane(r, 48)));
}

// Sums V values over the four 16-lane rows of a wave and spreads the V sums
// over the lanes: afterwards lane quarter q (lanes 16q .. 16q+15) holds in
// u[k] the sum of value q * V / 4 + k for the column (lane & 15).  Two rounds
// of gfx950 row swaps (v_permlane32_swap, then v_permlane16_swap), each
// exchanging two different values, take 3V/4 swaps and adds instead of 2V.
template <int V>
__device__ __forceinline__ void wave_rows_sum_spread(const float (&v)[V], float (&u)[V / 4]) {
  static_assert(V % 4 == 0, "four lane quarters");
  float t[V / 2];
#pragma unroll
  for (int k = 0; k < V / 2; ++k) {  // lanes 0-31: value k, 32-63: value k + V/2 (rows 0+2, 1+3)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + V / 2]), false, false);
    t[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < V / 4; ++k) {  // rows 0+1 / 2+3 of the pairs above
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(t[k]), __float_as_uint(t[k + V / 4]), false, false);
    u[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// Max / sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one column of the four
// 16-lane rows), left in all four: the same two row swaps.
__device__ __forceinline__ float quarters_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quarters_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A lane rescales its running sums only when a score exceeds its reference
// maximum by more than this (log2 domain): weights stay below 2^8, far from
// fp32 overflow, and the result is exact whatever the reference is.
constexpr float kRescaleGap = 8.f;

// Orders one wave's LDS accesses around an exchange between its lanes (the
// stores of some lanes before the loads of others, and those loads before the
// next stores to the same rows).  A wave's LDS instructions already execute in
// order; the fence makes the ordering part of the program rather than a
// property of the hardware, and the barrier keeps the compiler from moving
// accesses across it.  Neither emits an instruction.
__device__ __forceinline__ void wave_lds_exchange() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Device-coherent (agent scope) stores and loads of the split partials.  On
// gfx950 they carry the device scope bit, so a partial written on one XCD is
// read correctly on another without writing back or invalidating any L2.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float collect(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------
// element formats

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of a K/V row.  STREAM: the load carries the non-temporal hint.
// K/V rows are read once per pass; with the hint, loads whose instruction
// covers whole 128-byte lines stream about 14% faster (6.6 vs 5.7 TB/s for
// shuffled 4 KiB blocks), while half-line loads gain nothing or lose a little.
template <bool STREAM>
__device__ __forceinline__ uint4 kv_load(const char* p) {
  if constexpr (STREAM) {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// FP8 E4M3 (OCP encoding) to bf16 pairs and f32 pairs.  The gfx950
// conversion instructions decode this encoding exactly, and every E4M3 value
// is exact in bf16, so K can feed the bf16 dot instruction unchanged.  HI
// selects bytes 2..3 of the word instead of bytes 0..1.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& lo, float& hi) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  lo = f[0];
  hi = f[1];
}

// Register geometry of one K/V row.  A row is spread over LPR lanes; each lane
// holds NV 16-byte vectors of it.  Paged passes stream: four vectors per lane
// (bf16, f32) or two (FP8, whose freed tile registers carry a second pass of
// rows), so a lane's loads are large and its accumulators serve a long run of
// rows.  Ring passes take one 128-row tile per workgroup and are bound by
// latency: there a lane holds a single vector of each row (a bf16 d-128 row
// spans a whole 16-lane DPP row) over several passes, which keeps the lane's
// accumulators, and so the fold at the end of the pass, small.  Paged passes
// of GQA groups of 4 take half the vectors per lane and twice the passes (the
// same tile), so G accumulators of a lane's elements still fit two waves per
// SIMD without spilling; groups of 8 take a quarter of the vectors and twice
// the passes, a tile half as tall.  Passes of bf16 and FP8 groups of 4 and 8
// (MF) put both products on MFMA instead: lane l holds chunks 4j + l/16
// of row l % 16 of each 16-row pass (two passes per tile for FP8, so a tile
// still carries 64 KiB of K and V); each 8 of its elements (FP8 widened to
// bf16) are the A operand of one 16x16x32 bf16 form for S^T = K Q^T, the
// matching query elements its B operand; the scores come out as the B
// operand of the 16x16x16 form for O^T += V^T P^T, whose A operand (V
// transposed, as bf16) is read back from LDS.
template <int DT, int D, int SRC = kSrcPaged, int G = 1>
struct Geo {
  static constexpr int ES = DT == ODA_F32 ? 4 : (DT == ODA_BF16 ? 2 : 1);  // K/V element bytes
  static constexpr int QES = DT == ODA_F32 ? 4 : 2;                          // query element bytes
  static constexpr int ROW_BYTES = D * ES;
  static constexpr bool MF = DT != ODA_F32 && G >= 4;
  static constexpr bool WIDE = SRC == kSrcRing && DT != ODA_F32 && ROW_BYTES <= 16 * 16 && !MF;
  static constexpr int NARROW = WIDE || MF ? 1 : (G >= 8 ? 4 : (G >= 4 ? 2 : 1));  // divides NV
  static constexpr int PASSES = WIDE || MF ? 1 : (G >= 4 ? 2 : 1);                  // multiplies NP
  static constexpr int NV0 = WIDE ? 1 : MF ? D * ES / 64 : (DT == ODA_FP8_E4M3 ? 2 : 4) / NARROW;
  // Paged bf16 / f32 passes read whole 128-byte lines of a row per load
  // instruction (at least 8 lanes per row), with the non-temporal hint: loads
  // that cover half lines of twice as many rows stream about 12% slower and
  // gain nothing from the hint.  Fewer vectors per lane, more passes.  (FP8
  // rows would need a single vector per lane and four passes per tile, whose
  // per-row work costs more than the loads gain.)
  static constexpr int LINE_NV = ROW_BYTES >= 256 ? ROW_BYTES / 128 : 1;
  static constexpr int NV = SRC == kSrcPaged && !MF && ES >= 2 && NV0 > LINE_NV ? LINE_NV : NV0;  // 16-byte K/V vectors per lane per row
  static constexpr int LPR = ROW_BYTES / (16 * NV);  // lanes sharing a row
  static constexpr int RPP = kWave / LPR;            // rows per wave pass
  static constexpr int EPV = 16 / ES;                // elements per 16-byte K/V vector
  static constexpr int EPL = NV * EPV;               // elements per lane per row
  static constexpr int QV = EPL * QES / 16;          // 16-byte query vectors per lane per head
  static constexpr int QPV = QV / NV;                // query vectors per K/V vector
  static constexpr int NP = WIDE ? 128 / (kWavesPerGroup * RPP)
                                : (DT == ODA_FP8_E4M3 ? 2 : 1) * (MF ? 1 : PASSES) * (NV0 / NV);  // passes per tile
  static constexpr int TILE = kWavesPerGroup * NP * RPP;
  static_assert(LPR >= 2 && LPR <= 16, "row must span 2..16 lanes");
  static_assert(QV % NV == 0 && NP >= 1, "whole query vectors per K/V vector");
  static_assert(!MF || (LPR == 4 && RPP == 16 && G <= 16 && QV == NV * QPV && QES == 2),
                "MFMA pass: 16 rows of 4 lanes, bf16 queries");
};

// One element of a stored K/V row and of a query row, widened to f32.
template <int DT>
__device__ __forceinline__ float kv_elem(const char* row, int e) {
  if constexpr (DT == ODA_F32) {
    return reinterpret_cast<const float*>(row)[e];
  } else if constexpr (DT == ODA_BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[e] << 16);
  } else {
    float lo, hi;
    fp8x2_to_f32<false>((uint32_t) reinterpret_cast<const uint8_t*>(row)[e], lo, hi);
    return lo;
  }
}
template <int DT>
__device__ __forceinline__ float q_elem(const char* row, int e) {
  if constexpr (DT == ODA_F32) return reinterpret_cast<const float*>(row)[e];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[e] << 16);
}

// ----------------------------------------------------------------------------
// access-set index code (shared by every kernel that turns rows into positions)

// Ring state of a request just before decoding position t (1..t-1 committed).
struct RingState {
  int32_t t, s, w;
  int32_t c;     // latest committed position (t - 1)
  int32_t r;     // window slot offset of position c, valid when c > s
};

__device__ __forceinline__ RingState ring_state(int32_t t, int32_t s, int32_t w) {
  RingState st;
  st.t = t;
  st.s = s;
  st.w = w;
  st.c = t - 1;
  st.r = st.c > s ? (st.c - s - 1) % w : 0;
  return st;
}

// Position the one-by-one commits left in slot j (0 if none), and whether it
// belongs to the Local set of t.  Window slot k = j - s holds the latest
// committed position p > s with (p - s - 1) mod w == k.
__device__ __forceinline__ int32_t ring_slot_position(const RingState& st, int32_t j, bool& in_local) {
  if (j < st.s) {
    const int32_t p = j + 1;
    in_local = p <= st.c;
    return in_local ? p : 0;
  }
  if (st.c <= st.s) {
    in_local = false;
    return 0;
  }
  int32_t back = st.r - (j - st.s);
  if (back < 0) back += st.w;
  const int32_t p = st.c - back;
  if (p <= st.s) {
    in_local = false;
    return 0;
  }
  in_local = p >= st.t - st.w + 1;  // excludes only position t - w
  return p;
}

// Rows a ring pass scans: the filled prefix of the ring.
__device__ __forceinline__ int32_t ring_rows(int32_t t, int32_t slots) {
  return min(slots, t - 1);
}

// Positions a paged pass reads (the current token t excluded), as up to three
// disjoint ascending closed intervals.
struct Intervals {
  int32_t lo[3];
  int32_t n[3];
  int32_t total;
};

__device__ __forceinline__ Intervals paged_intervals(const RowSpec& rs, int32_t t, int64_t fa, int64_t fb) {
  Intervals iv;
  const int32_t last = t - 1;
  if (!rs.focus) {
    iv.lo[0] = 1;
    iv.n[0] = max(last, 0);
    iv.lo[1] = iv.lo[2] = 1;
    iv.n[1] = iv.n[2] = 0;
    iv.total = iv.n[0];
    return iv;
  }
  // S^L_t U [a, b), minus t: sinks, focus region, window -- then sort and merge.
  int32_t lo[3], hi[3];
  lo[0] = 1;
  hi[0] = min(rs.sink, last);
  const int64_t a = fa < 1 ? 1 : fa;
  const int64_t bb = (fb - 1) < last ? (fb - 1) : last;
  lo[1] = (int32_t)(a > (int64_t)last + 1 ? (int64_t)last + 1 : a);
  hi[1] = (int32_t)(bb < 0 ? 0 : bb);
  lo[2] = max(1, t - rs.window + 1);
  hi[2] = last;
  for (int i = 0; i < 3; ++i)
    for (int k = 0; k + 1 < 3 - i; ++k)
      if (lo[k] > lo[k + 1]) {
        int32_t x = lo[k]; lo[k] = lo[k + 1]; lo[k + 1] = x;
        x = hi[k]; hi[k] = hi[k + 1]; hi[k + 1] = x;
      }
  int32_t m = 0;
  int32_t mlo[3], mhi[3];
  for (int k = 0; k < 3; ++k) {
    if (hi[k] < lo[k]) continue;  // empty
    if (m > 0 && lo[k] <= mhi[m - 1] + 1) {
      mhi[m - 1] = max(mhi[m - 1], hi[k]);
    } else {
      mlo[m] = lo[k];
      mhi[m] = hi[k];
      ++m;
    }
  }
  iv.total = 0;
  for (int k = 0; k < 3; ++k) {
    if (k < m) {
      iv.lo[k] = mlo[k];
      iv.n[k] = mhi[k] - mlo[k] + 1;
    } else {
      iv.lo[k] = 1;
      iv.n[k] = 0;
    }
    iv.total += iv.n[k];
  }
  return iv;
}

__device__ __forceinline__ int32_t interval_position(const Intervals& iv, int32_t row) {
  if (row < iv.n[0]) return iv.lo[0] + row;
  row -= iv.n[0];
  if (row < iv.n[1]) return iv.lo[1] + row;
  row -= iv.n[1];
  return iv.lo[2] + row;
}

// Splitting n_rows over `splits` workgroups in whole tiles.
// Rows [0, n) of a pass go to `splits` contiguous ranges made of whole units of
// kSplitRowUnit rows, as even as whole units allow (range sizes differ by one
// unit at most, so no workgroup of a launch carries a whole tile more than
// another).  The larger ranges come first: the last split, which is
// dispatched last and merges, takes the fewest rows.  The first `used` ranges
// are non-empty; `split` < `used` gets [begin, end).
constexpr int32_t kSplitRowUnit = 16;
// Tail-pool tiles per split (paged passes over long ranges).  At 128K, bf16
// group 2: the pool saves 2.6 us per Full launch over static splits alone,
// and pools of 6, 10 and 16 tiles per split measured no faster than 3.  (At
// 16K, where a split has 4 tiles, a pool of one tile per split made the
// launch 1.5 us slower: a pool tile costs a claim and a full round trip.)
constexpr int32_t kPoolTilesPerSplit = 3;
// The pool's block ids are staged in LDS when the pool starts; the pool is
// sized so that they fit.
constexpr int32_t kPoolBlkMax = 2048;
// Rows of the tail pool of a paged pass (0: none).  Its rows, plus what the
// whole-unit rounding of the static shares leaves over (under
// kSplitRowUnit rows per split), span at most kPoolBlkMax blocks.
__device__ __forceinline__ int32_t pool_rows_of(int32_t splits, int32_t block_shift, int32_t tile) {
  const int64_t cap = ((int64_t)(kPoolBlkMax - 2) << block_shift) - (int64_t)kSplitRowUnit * splits;
  int64_t rows = (int64_t)kPoolTilesPerSplit * splits * tile;
  if (rows > cap) rows = cap / tile * tile;
  return rows >= tile ? (int32_t)rows : 0;
}
// Takes the next pool tile: a relaxed device-scope increment of the counter.
__device__ __forceinline__ int32_t claim_next(int32_t* counter) {
  return (int32_t)__builtin_amdgcn_atomic_inc32(reinterpret_cast<uint32_t*>(counter), 0xFFFFFFFFu, __ATOMIC_RELAXED,
                                                "agent");
}
__device__ __forceinline__ void split_rows(int32_t n, int32_t splits, int32_t split, int32_t& used,
                                           int32_t& begin, int32_t& end) {
  const int32_t units = (n + kSplitRowUnit - 1) / kSplitRowUnit;
  used = units < splits ? units : splits;
  if (used < 1) used = 1;
  const int32_t base = units / used, rem = units % used;
  begin = (split * base + min(split, rem)) * kSplitRowUnit;
  end = split + 1 >= used ? n : ((split + 1) * base + min(split + 1, rem)) * kSplitRowUnit;
}

// ----------------------------------------------------------------------------
// which request a workgroup serves

// The z-th request (ascending) whose score exceeds theta, found by wave ballots;
// every wave computes the same answer.  -1 when fewer than z+1 fired.  Also
// returns the request's committed length, read in the same round trip.
__device__ __forceinline__ int32_t ballot_request(const AttnParams& P, int32_t slot, int32_t& committed) {
  const int lane = threadIdx.x & (kWave - 1);
  int32_t seen = 0;
  for (int32_t c = 0; c < P.batch; c += kWave) {
    const int32_t b = c + lane;
    const int32_t r = b < P.batch ? b : P.batch - 1;  // both words in one round trip
    const int32_t stored = P.seq_len[r];
    const float score = P.score[r];
    __builtin_amdgcn_sched_barrier(0);
    const int32_t len = b < P.batch ? stored : -1;
    const bool fire = len >= 0 && score > P.theta;  // NaN never fires
    const uint64_t mask = __ballot(fire);
    const int32_t n = __popcll(mask);
    if (slot < seen + n) {
      const uint64_t below = mask & ((1ull << lane) - 1ull);
      const uint64_t hit = __ballot(fire && __popcll(below) == slot - seen);
      const int src = __ffsll((unsigned long long)hit) - 1;
      committed = __shfl(len, src, kWave);
      return c + src;
    }
    seen += n;
  }
  return -1;
}

// Writes the compacted list of fired requests (ascending, then -1) and its length.
__device__ __forceinline__ void write_call_list(const AttnParams& P) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  int32_t seen = 0;
  for (int32_t c = 0; c < P.batch; c += kWave) {
    const int32_t b = c + lane;
    const int32_t r = b < P.batch ? b : P.batch - 1;  // both words in one round trip
    const int32_t len = P.seq_len[r];
    const float score = P.score[r];
    __builtin_amdgcn_sched_barrier(0);
    const bool fire = b < P.batch && len >= 0 && score > P.theta;
    const uint64_t mask = __ballot(fire);
    const uint64_t below = mask & ((1ull << lane) - 1ull);
    if (fire && P.call_list_out) P.call_list_out[seen + __popcll(below)] = b;
    seen += __popcll(mask);
  }
  if (P.call_list_out)
    for (int32_t i = seen + lane; i < P.batch; i += kWave) P.call_list_out[i] = -1;
  if (lane == 0 && P.call_count_out) *P.call_count_out = seen;
}

// ----------------------------------------------------------------------------
// merge of the split partials (run by one workgroup)

// A partial slot reads kPartialEmpty (a signalling NaN, which no arithmetic
// result ever is) from the moment a merge has consumed it until a workgroup
// of a later launch stores its partial there.  The merging workgroup of a
// launch whose workgroups are all resident at once therefore needs no flag or
// counter: it reads the slots and reads again those still empty.
constexpr uint32_t kPartialEmpty = 0x7FA5A5A5u;
__device__ __forceinline__ bool slot_empty(float x) { return __float_as_uint(x) == kPartialEmpty; }

constexpr int kMergeBatch = 32;  // partials loaded per round by one output thread

// One thread per output element (h, e) (two when G * d exceeds the
// workgroup); a wave serves one head at a time.  Partials
// 0..n_mem-1 are read from the workspace in rounds of up to kMergeBatch:
// lane i loads (m, l) of partial i of the round (one 8-byte load), every lane
// loads its element of each partial's o, the round's maximum and weights come
// from lane exchanges, and the weights reach every lane by lane reads.  With
// `poll`, a round is read again (by the whole wave) while any of its values is
// still empty.  `own_o` / `own_ml` (LDS, may be null) is one more partial,
// the merging workgroup's own.  Each round's slots are left empty for the
// next launch as soon as they are read.  Returns false (and sets ODA_DEVERR_MERGE_WAIT) if polling gives up.
// No LDS writes, no barrier.
template <int DT, int D, int G>
__device__ __forceinline__ bool merge_output(const AttnParams& P, int32_t b, int32_t g, int32_t n_mem, bool poll,
                             const float* own_o, const float* own_ml, int tid, int32_t spin_limit) {
  const int lane = tid & (kWave - 1);
  const int h = tid / D, e = tid % D;
  const int64_t head0 = (int64_t)b * P.Hq + (int64_t)g * G;
  // (m, l) is stored once per wave of a head (D / 64 copies), so each wave
  // reads, checks and empties its own copy.
  constexpr int kCopies = D / kWave;
  const int half = e / kWave;
  float* ml = P.part_ml + (head0 + h) * P.splits * 2 * kCopies + 2 * half;
  float* po = P.part_o + (head0 + h) * P.splits * D + e;
  const float empty = __uint_as_float(kPartialEmpty);
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int32_t base = 0; base < n_mem; base += kMergeBatch) {
    const int32_t n = n_mem - base < kMergeBatch ? n_mem - base : kMergeBatch;
    // Branch-free: slots past the round's end re-read its last partial (their
    // weights are zero below), so all loads leave back to back.
    float x[kMergeBatch];
    float mi, li;
    for (int32_t spin = 0;; ++spin) {
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) x[i] = collect(po + (int64_t)(base + (i < n ? i : n - 1)) * D);
      mi = -INFINITY;
      li = 0.f;
      if (lane < n) {
        const uint64_t w2 = __hip_atomic_load(reinterpret_cast<uint64_t*>(ml + 2 * kCopies * (base + lane)),
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mi = __uint_as_float((uint32_t)w2);
        li = __uint_as_float((uint32_t)(w2 >> 32));
      }
      if (!poll) break;
      bool missing = slot_empty(mi) || slot_empty(li);
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) missing = missing || slot_empty(x[i]);
      if (!__any(missing)) break;
      if (spin == spin_limit) {
        if (lane == 0) atomicOr(P.err, (uint32_t)ODA_DEVERR_MERGE_WAIT);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    {
      // The round's slots are read: this wave leaves what it read empty for
      // the next pass, its 64 elements of each of the n rows of o and its copy
      // of (m, l).  Device-scope stores, like the partials themselves: no
      // dirty line of them stays in this XCD's L2, where a later write-back
      // could land on a partial stored after them.
      float* ro = P.part_o + ((head0 + h) * P.splits + base) * D + half * kWave;
      for (int32_t i = 0; i < n; ++i) publish(ro + (int64_t)i * D + lane, empty);
      if (lane < n) {
        publish(ml + 2 * kCopies * (base + lane), empty);
        publish(ml + 2 * kCopies * (base + lane) + 1, empty);
      }
    }
    const float m_new = fmaxf(M, wave_max(mi));
    const float keep = M == -INFINITY ? 0.f : fast_exp2(M - m_new);
    const float wi = mi == -INFINITY ? 0.f : fast_exp2(mi - m_new);
    L = fmaf(L, keep, wave_sum(wi * li));
    float part[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)  // lanes >= n hold weight 0
      part[i & 3] = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), i)), x[i], part[i & 3]);
    acc = fmaf(acc, keep, (part[0] + part[1]) + (part[2] + part[3]));
    M = m_new;
  }
  if (own_o != nullptr) {
    const float mo = own_ml[2 * h], lo = own_ml[2 * h + 1];
    const float m_new = fmaxf(M, mo);
    const float keep = M == -INFINITY ? 0.f : fast_exp2(M - m_new);
    const float wo = mo == -INFINITY ? 0.f : fast_exp2(mo - m_new);
    L = fmaf(L, keep, wo * lo);
    acc = fmaf(acc, keep, wo * own_o[tid]);
    M = m_new;
  }
  P.out[(head0 + h) * D + e] = acc * (__builtin_amdgcn_rcpf(L) * P.v_scale);
  if (P.lse != nullptr && e == 0) P.lse[head0 + h] = (M + __log2f(L)) * kLn2;
  return true;
}

template <int DT, int D, int G>
__device__ __forceinline__ bool merge_and_write(const AttnParams& P, int32_t b, int32_t g, int32_t n_mem, bool poll,
                                const float* own_o, const float* own_ml, int32_t spin_limit = kMergeSpinLimit) {
  static_assert(D % kWave == 0, "one head per wave");
  for (int tid = threadIdx.x; tid < G * D; tid += kGroupThreads)
    if (!merge_output<DT, D, G>(P, b, g, n_mem, poll, own_o, own_ml, tid, spin_limit)) return false;
  return true;
}

// ----------------------------------------------------------------------------
// one attention pass of one layer: split-K partials + last-workgroup merge

// SKIP: passes without rows of this split are skipped by wave-uniform branches
// (the host asks for it when the splits are shorter than a tile, and for paged
// passes).  Without it, a ring pass that loops over many tiles keeps its loads
// in flight across the joins.
// WITHHOLD (the test of the merge's failure path only): split `withheld`
// stores no partial and the merging workgroup gives up after `spin_limit`
// re-reads of the partial slots.
template <int DT, int D, int G, int SRC, bool BALLOT, bool SKIP, bool WITHHOLD = false>
__device__ __forceinline__ void attention_pass(const AttnParams& P, int32_t withheld = -1,
                                               int32_t spin_limit = kMergeSpinLimit) {
  using Gm = Geo<DT, D, SRC, G>;
  constexpr int LPR = Gm::LPR, RPP = Gm::RPP, EPV = Gm::EPV, EPL = Gm::EPL, NP = Gm::NP;
  constexpr int NV = Gm::NV, QV = Gm::QV, QPV = Gm::QPV;
  constexpr int TILE = Gm::TILE;
  constexpr int ES = Gm::ES, QES = Gm::QES;
  ODA_PHASE(0);
  ODA_PHASE_XCC();

  // Paged Full passes with the tail pool, no focus region: when the context
  // fills the block table to within the pool and the workgroup's request
  // turns out to be request blockIdx.z (batch 1, or every request firing), the
  // static share of every split is fixed by the table's capacity alone, so the
  // block ids of this split's first tile are read here, in the same round trip
  // as the request's state.
  int32_t spec_blk[NP];
  int32_t spec_S = 0;
  if constexpr (SRC == kSrcPaged) {
    const int32_t pool_rows = pool_rows_of(P.splits, P.block_shift, TILE);
    const int32_t S = ((P.capacity - pool_rows) / P.splits) & ~(kSplitRowUnit - 1);
    if (!P.rows.focus && P.claims != nullptr && pool_rows > 0 && S >= TILE && P.capacity >= 2 * pool_rows) {
      spec_S = S;
      const int32_t* bt = P.block_table + (int64_t)blockIdx.z * P.max_blocks;
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      const int rr = Gm::MF ? (int)(threadIdx.x % RPP) : (int)(threadIdx.x & (kWave - 1)) / LPR;
#pragma unroll
      for (int i = 0; i < NP; ++i)  // rows < P.splits * S < capacity: inside the table row
        spec_blk[i] = bt[((int32_t)blockIdx.x * S + (i * kWavesPerGroup + w) * RPP + rr) >> P.block_shift];
    }
  }

  // The request this workgroup serves and its committed length (-1 = none).
  int32_t b;
  int32_t committed = -1;
  if constexpr (BALLOT) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) write_call_list(P);
    b = ballot_request(P, blockIdx.z, committed);
  } else if (P.gate_mode == kGateList) {
    // The count and this slot's entries (written with the list by the gate)
    // are read in one round trip: every slot below the launch's batch exists,
    // and entries past the count are not used.  (The three pointers sit in one
    // 64-byte block of the kernel arguments, loaded with the first batch.)
    const int32_t count = *P.call_count;
    const int32_t listed = P.call_list[blockIdx.z];
    const int32_t len = P.call_len[blockIdx.z];
    __builtin_amdgcn_sched_barrier(0);  // all three loads leave before the first wait
    const bool in_list = (int32_t)blockIdx.z < count;
    b = in_list ? listed : -1;
    committed = in_list ? len : -1;
  } else {
    b = blockIdx.z;
  }
  if (b < 0) return;
  const int32_t g = blockIdx.y;
  const int32_t split = blockIdx.x;

  // Ring passes scan every slot of the ring whatever t is, so their first tile
  // loads need no per-request state and go out before seq_len arrives; which
  // slots belong to S^L_t is decided per row once t is known.  Paged passes
  // need t (and the block table) to know what to read.
  int32_t t = 0;
  RingState rst{};
  Intervals iv{};
  int32_t n_rows;
  if constexpr (SRC == kSrcRing) {
    n_rows = P.rows.ring_slots;
  } else {
    if (P.gate_mode == kGateAll) committed = P.seq_len[b];
    if (committed < 0) return;
    ODA_PHASE(1);
    t = committed + 1;
    if (t - 1 > P.capacity) {
      if (threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) atomicOr(P.err, (uint32_t)ODA_DEVERR_CAPACITY);
      return;
    }
    int64_t fa = 0, fb = 0;
    if (P.rows.focus) {
      fa = P.focus_range[2 * b];
      fb = P.focus_range[2 * b + 1];
    }
    iv = paged_intervals(P.rows, t, fa, fb);
    n_rows = iv.total;
  }
  // Row n_rows is the current token t, read from k_cur / v_cur: it is
  // processed like any other row, by the last split (or, with the pool, by the
  // workgroup that takes the last pool tile).
  // Paged passes over long ranges (no focus region) keep a pool of tail
  // tiles, kPoolTilesPerSplit per split, at the end of the range: the splits
  // divide rows [0, n_static) statically and then take pool tiles from a
  // per-(request, KV head) counter, so workgroups that stream faster than
  // others take more of the tail.
  const int32_t n_all = n_rows + 1;
  int32_t n_static = n_all;
  int32_t used, row_begin, row_end;
  const bool spec_hit = spec_S > 0 && b == (int32_t)blockIdx.z && n_all > P.splits * spec_S + TILE;
  if (spec_hit) {  // the same for every workgroup of this (request, KV head)
    n_static = P.splits * spec_S;
    used = P.splits;
    row_begin = split * spec_S;
    row_end = row_begin + spec_S;
  } else {
    if constexpr (SRC == kSrcPaged) {
      const int32_t pool_rows = pool_rows_of(P.splits, P.block_shift, TILE);
      if (!P.rows.focus && P.claims != nullptr && pool_rows > 0 && n_all >= 2 * pool_rows)
        n_static = (n_all - pool_rows) & ~(kSplitRowUnit - 1);
    }
    split_rows(n_static, P.splits, split, used, row_begin, row_end);
    if (split >= used) return;
  }
  // Tiles of this split: rows row_begin + k * TILE ...; rows at or past row_end
  // belong to the next split and stay out of the sums.
  const int32_t n_tiles = (row_end - row_begin + TILE - 1) / TILE;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // A lane's row within its wave's pass and its chunk group within the row.
  const int sub = Gm::MF ? lane / RPP : lane % LPR;
  const int rrow = Gm::MF ? lane % RPP : lane / LPR;

  // Query heads g*G .. g*G+G-1, in this lane's element slots.
  // Query vector j covers the elements of K/V vector j / QPV.
  // (MF: the B operand of S^T = K Q^T, head lane % 16, zero past the group.)
  constexpr int QH = Gm::MF ? 1 : G;
  uint4 qv[QH][QV];
  if constexpr (Gm::MF) {
    const char* qbase = static_cast<const char*>(P.q) + ((int64_t)b * P.Hq + (int64_t)g * G) * D * QES;
    const int hq = lane % 16;
#pragma unroll
    for (int j = 0; j < QV; ++j)
      qv[0][j] = hq < G ? *reinterpret_cast<const uint4*>(qbase + (int64_t)hq * D * QES +
                                                          ((j / QPV) * LPR + sub) * EPV * QES + (j % QPV) * 16)
                        : make_uint4(0, 0, 0, 0);
  } else {
    const char* qbase = static_cast<const char*>(P.q) + ((int64_t)b * P.Hq + (int64_t)g * G) * D * QES;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < QV; ++j)
        qv[h][j] = *reinterpret_cast<const uint4*>(qbase + (int64_t)h * D * QES +
                                                   ((j / QPV) * LPR + sub) * EPV * QES + (j % QPV) * 16);
  }

  const char* kbase = static_cast<const char*>(P.k_base);
  const char* vbase = static_cast<const char*>(P.v_base);
  int64_t ring_head_off = 0;
  if constexpr (SRC == kSrcRing)
    ring_head_off = (((int64_t)b * P.Hkv + g) * P.rows.ring_slots) * D * ES;
  const int32_t* btab = P.block_table + (int64_t)b * P.max_blocks;
  const int32_t bmask = (1 << P.block_shift) - 1;
  const int64_t cur_off = ((int64_t)b * P.Hkv + g) * D * ES;

  constexpr int OE = Gm::MF ? 1 : EPL;
  float m_run[G], l_acc[G], o[G][OE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_acc[h] = 0.f;
#pragma unroll
    for (int e = 0; e < OE; ++e) o[h][e] = 0.f;
  }
  // MF: O^T tiles (lane l: elements 16 mi + 4 (l / 16) + r of head l % 16),
  // and the running reference and weight sum of head l % 16, the same in the
  // four lanes of the head.  V rows are staged per wave in LDS (row stride
  // VST bytes: the four row quarters of a transposed read fall on different
  // banks).
  constexpr int MT = Gm::MF ? D / 16 : 1;
  constexpr int VST = 2 * D + 16;
  f32x4_t acc_mf[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) acc_mf[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_mf = -INFINITY, l_mf = 0.f;
  __shared__ __align__(16) char s_vt[Gm::MF ? kWavesPerGroup * 16 * VST : 16];

  // Tile registers: K and V of NP passes plus their validity.  Two sets
  // ping-pong so the loads of tile i+1 are in flight while tile i is reduced.
  struct TileRegs {
    uint4 k[NP][NV];
    uint4 v[NP][NV];
    bool valid[NP];  // paged: row in the pass; ring: row inside the ring (membership checked later)
    bool live[NP];   // wave-uniform: the pass has rows of this split
    int32_t row[NP];
  };
  // Paged rows: the physical block of each lane's row, looked up two tiles
  // before its K/V loads so the dependent block-table read is never waited on.
  // -1 marks a row outside the pass (or a block id the table gets wrong).
  struct BlockIds {
    int32_t blk[NP];
    bool ok[NP];  // the row is in the pass (blk was read for it)
  };
  // Paged passes read every lane's table entry and K/V rows unconditionally:
  // a row outside the pass reads position 1's entry and the current token's
  // row, and is masked when the tile is reduced.  Loads on conditional paths
  // make the compiler wait for every outstanding load before the next one, so
  // with them a wave keeps one tile in flight instead of two.
  uint32_t bad_blk = 0;
  auto resolve_blocks = [&](int32_t tile, BlockIds& B, int32_t slot) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      B.blk[i] = -1;
      B.ok[i] = false;
      if constexpr (SRC == kSrcPaged) {
        const int32_t row = row_begin + tile * TILE + (i * kWavesPerGroup + slot) * RPP + rrow;
        const bool in = tile < n_tiles && row < row_end && row < n_rows;
        const int32_t p = interval_position(iv, in ? row : 0);
        B.blk[i] = btab[(p - 1) >> P.block_shift];
        B.ok[i] = in;
      }
    }
  };
  auto load_tile = [&](int32_t tile, const BlockIds& B, TileRegs& R, int32_t slot) {
    if constexpr (SRC == kSrcPaged) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int32_t pass0 = row_begin + tile * TILE + (i * kWavesPerGroup + slot) * RPP;
        const int32_t row = pass0 + rrow;
        R.row[i] = row;
        R.live[i] = !SKIP || pass0 < row_end;
        const int32_t blk = B.blk[i];
        const bool blk_ok = blk >= 0 && (int64_t)blk < P.num_blocks;
        bad_blk |= B.ok[i] && !blk_ok;
        const bool from_cache = B.ok[i] && blk_ok;
        R.valid[i] = from_cache || (row == n_rows && row < row_end);
        const int32_t r0 = interval_position(iv, from_cache ? row : 0) - 1;
        const char* kb = from_cache ? kbase : static_cast<const char*>(P.k_cur);
        const char* vb = from_cache ? vbase : static_cast<const char*>(P.v_cur);
        const int64_t off =
            from_cache ? ((((int64_t)g * P.num_blocks + blk) << P.block_shift) + (r0 & bmask)) * D * ES : cur_off;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          // non-temporal where a load instruction covers whole 128-byte lines
          constexpr bool kStream = LPR * 16 >= 128;
          R.k[i][j] = kv_load<kStream>(kb + off + (j * LPR + sub) * 16);
          R.v[i][j] = kv_load<kStream>(vb + off + (j * LPR + sub) * 16);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int32_t row = row_begin + tile * TILE + (i * kWavesPerGroup + wave) * RPP + rrow;
      R.row[i] = row;
      // Pass i of a tile covers rows i*8*RPP .. (i+1)*8*RPP-1 across the 8 waves, so
      // a split shorter than a tile leaves whole passes empty in every wave and
      // both waves of a SIMD skip them.
      if constexpr (SKIP) {
        R.live[i] = row_begin + tile * TILE + (i * kWavesPerGroup + wave) * RPP < row_end;
        if (!R.live[i]) {
          R.valid[i] = false;
          continue;
        }
      }
      bool ok = row < row_end;  // row_end <= n_rows + 1
      const char* kb = kbase;
      const char* vb = vbase;
      int64_t off = 0;
      if (row == n_rows) {
        kb = static_cast<const char*>(P.k_cur);
        vb = static_cast<const char*>(P.v_cur);
        off = cur_off;
      } else {
        off = ring_head_off + (int64_t)row * D * ES;
      }
      R.valid[i] = ok;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (ok) {
          R.k[i][j] = kv_load<true>(kb + off + (j * LPR + sub) * 16);
          R.v[i][j] = kv_load<true>(vb + off + (j * LPR + sub) * 16);
        } else {
          R.k[i][j] = make_uint4(0, 0, 0, 0);
          R.v[i][j] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto process_tile = [&](TileRegs& R) {
    if constexpr (Gm::MF) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {  // 16 rows of each wave per pass
        if (SKIP && !R.live[i]) continue;
        if constexpr (SRC == kSrcRing) {  // membership in S^L_t: other slots may hold anything
          bool in_local = R.valid[i] && R.row[i] == n_rows;
          if (R.valid[i] && !in_local) ring_slot_position(rst, R.row[i], in_local);
          R.valid[i] = in_local;
#pragma unroll
          for (int j = 0; j < NV; ++j)
            if (!in_local) R.v[i][j] = make_uint4(0, 0, 0, 0);
        }
        // S^T = K Q^T: lane l gets the scores of rows 4 (l / 16) + r of head l % 16
        // (a row outside the sums may hold anything; its scores are dropped).
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < QV; ++j) {  // the lane's row elements 8j .. 8j + 7
          uint4 ka = R.k[i][j / QPV];
          if constexpr (DT == ODA_FP8_E4M3) {
            const uint32_t w0 = j % 2 ? ka.z : ka.x, w1 = j % 2 ? ka.w : ka.y;
            ka = make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                            fp8x2_to_bf16x2<true>(w1));
          }
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                       __builtin_bit_cast(bf16x8_t, qv[0][j]), sc, 0, 0, 0);
        }
        // The pass's V rows go to LDS as bf16 rows.
        char* vt = s_vt + wave * 16 * VST;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          char* dst = vt + rrow * VST + (j * LPR + sub) * EPV * 2;
          // a paged row outside the sums may hold anything (pool loads are unconditional)
          const uint4 vv = SRC == kSrcPaged && !R.valid[i] ? make_uint4(0, 0, 0, 0) : R.v[i][j];
          if constexpr (DT == ODA_FP8_E4M3) {
            const uint4 w = vv;
            *reinterpret_cast<uint4*>(dst) = make_uint4(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                                                        fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y));
            *reinterpret_cast<uint4*>(dst + 16) = make_uint4(fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z),
                                                             fp8x2_to_bf16x2<false>(w.w), fp8x2_to_bf16x2<true>(w.w));
          } else {
            *reinterpret_cast<uint4*>(dst) = vv;
          }
        }
        wave_lds_exchange();  // the pass's V rows are in LDS before any lane reads them transposed
        const uint64_t vm = __ballot(R.valid[i]);  // bit r: row r of the pass is in the sums
        const int q4 = (lane >> 4) * 4;
        float s[4];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[r] = (vm >> (q4 + r)) & 1 ? sc[r] * P.scale_log2 : -INFINITY;
          mx = fmaxf(mx, s[r]);
        }
        mx = quarters_max(mx);
        if (mx > m_mf + kRescaleGap) {
          const float alpha = m_mf == -INFINITY ? 0.f : fast_exp2(m_mf - mx);
          l_mf *= alpha;
#pragma unroll
          for (int mi = 0; mi < MT; ++mi) acc_mf[mi] *= alpha;
          m_mf = mx;
        }
        // P^T as a sum of two bf16 parts (the second holds what rounding the
        // first lost), so the weights keep about 16 bits in the products.
        i16x4_t ph, pl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float w = s[r] == -INFINITY ? 0.f : fast_exp2(s[r] - m_mf);
          const __bf16 wh = (__bf16)w;
          ph[r] = __builtin_bit_cast(short, wh);
          pl[r] = __builtin_bit_cast(short, (__bf16)(w - (float)wh));
          l_mf += w;
        }
        // O^T += V^T P^T, 16 elements at a time: lane l reads element
        // 16 mi + l % 16 of rows 4 (l / 16) + r.
        const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vt);
        i16x4_t va[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
          for (int r = 0; r < 4; ++r) va[mi][r] = (short)vt16[(q4 + r) * (VST / 2) + 16 * mi + lane % 16];
          acc_mf[mi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[mi], ph, acc_mf[mi], 0, 0, 0);
        }
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          acc_mf[mi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[mi], pl, acc_mf[mi], 0, 0, 0);
        wave_lds_exchange();  // every transposed read is done before the next pass overwrites the rows
      }
    } else {
    if constexpr (SRC == kSrcRing) {
      // Membership in S^L_t; rows outside it never reach the sums (slots not
      // yet written may hold anything, so their values are replaced by zeros).
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (SKIP && !R.live[i]) continue;
        bool in_local = R.valid[i] && R.row[i] == n_rows;  // the current token
        if (R.valid[i] && !in_local) ring_slot_position(rst, R.row[i], in_local);
        R.valid[i] = in_local;
#pragma unroll
        for (int j = 0; j < NV; ++j)
          if (!in_local) R.v[i][j] = make_uint4(0, 0, 0, 0);
      }
    }
    // scores s = scale*log2(e) * <q_h, k_row>
    float s[NP][G];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (SKIP && !R.live[i]) continue;
      // FP8 keys become bf16 pairs once per row, shared by the G heads.
      uint32_t kb[DT == ODA_FP8_E4M3 ? 2 * 4 * NV : 1];
      if constexpr (DT == ODA_FP8_E4M3) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const uint32_t w4[4] = {R.k[i][j].x, R.k[i][j].y, R.k[i][j].z, R.k[i][j].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            kb[8 * j + 2 * c] = fp8x2_to_bf16x2<false>(w4[c]);
            kb[8 * j + 2 * c + 1] = fp8x2_to_bf16x2<true>(w4[c]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const uint4 kk = R.k[i][j];
          const uint4 qq = qv[h][j * QPV];
          if constexpr (DT == ODA_FP8_E4M3) {
            const uint4 q1 = qv[h][j * QPV + 1];
            acc = dot2_bf16(kb[8 * j + 0], qq.x, acc);
            acc = dot2_bf16(kb[8 * j + 1], qq.y, acc);
            acc = dot2_bf16(kb[8 * j + 2], qq.z, acc);
            acc = dot2_bf16(kb[8 * j + 3], qq.w, acc);
            acc = dot2_bf16(kb[8 * j + 4], q1.x, acc);
            acc = dot2_bf16(kb[8 * j + 5], q1.y, acc);
            acc = dot2_bf16(kb[8 * j + 6], q1.z, acc);
            acc = dot2_bf16(kb[8 * j + 7], q1.w, acc);
          } else if constexpr (DT == ODA_BF16) {
            acc = dot2_bf16(kk.x, qq.x, acc);
            acc = dot2_bf16(kk.y, qq.y, acc);
            acc = dot2_bf16(kk.z, qq.z, acc);
            acc = dot2_bf16(kk.w, qq.w, acc);
          } else {
            acc = fmaf(__uint_as_float(kk.x), __uint_as_float(qq.x), acc);
            acc = fmaf(__uint_as_float(kk.y), __uint_as_float(qq.y), acc);
            acc = fmaf(__uint_as_float(kk.z), __uint_as_float(qq.z), acc);
            acc = fmaf(__uint_as_float(kk.w), __uint_as_float(qq.w), acc);
          }
        }
        acc = lane_group_sum<LPR>(acc);
        s[i][h] = R.valid[i] ? acc * P.scale_log2 : -INFINITY;
      }
    }

    // Per-lane reference maximum (the LPR lanes of a row agree on it): move it
    // only when a score would push a weight past 2^kRescaleGap.
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (SKIP && !R.live[i]) continue;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (s[i][h] > m_run[h] + kRescaleGap) {
          const float alpha = m_run[h] == -INFINITY ? 0.f : fast_exp2(m_run[h] - s[i][h]);
          l_acc[h] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
          m_run[h] = s[i][h];
        }
      }
    }

    // p = exp2(s - m); o += p * v
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (SKIP && !R.live[i]) continue;
      float pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pr[h] = R.valid[i] ? fast_exp2(s[i][h] - m_run[h]) : 0.f;
        l_acc[h] += pr[h];
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        // a paged row outside the sums may hold anything (pool loads are unconditional)
        const uint4 vv = SRC == kSrcPaged && !R.valid[i] ? make_uint4(0, 0, 0, 0) : R.v[i][j];
        const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (DT == ODA_FP8_E4M3) {
            float v0, v1, v2, v3;
            fp8x2_to_f32<false>(w4[c], v0, v1);
            fp8x2_to_f32<true>(w4[c], v2, v3);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              o[h][j * EPV + 4 * c] = fmaf(pr[h], v0, o[h][j * EPV + 4 * c]);
              o[h][j * EPV + 4 * c + 1] = fmaf(pr[h], v1, o[h][j * EPV + 4 * c + 1]);
              o[h][j * EPV + 4 * c + 2] = fmaf(pr[h], v2, o[h][j * EPV + 4 * c + 2]);
              o[h][j * EPV + 4 * c + 3] = fmaf(pr[h], v3, o[h][j * EPV + 4 * c + 3]);
            }
          } else if constexpr (DT == ODA_BF16) {
            const float v0 = bf16_lo(w4[c]);
            const float v1 = bf16_hi(w4[c]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              o[h][j * EPV + 2 * c] = fmaf(pr[h], v0, o[h][j * EPV + 2 * c]);
              o[h][j * EPV + 2 * c + 1] = fmaf(pr[h], v1, o[h][j * EPV + 2 * c + 1]);
            }
          } else {
            const float v0 = __uint_as_float(w4[c]);
#pragma unroll
            for (int h = 0; h < G; ++h) o[h][j * EPV + c] = fmaf(pr[h], v0, o[h][j * EPV + c]);
          }
        }
      }
    }
    }
  };

  // Element by element (an aggregate copy can leave the tiles in scratch memory).
  auto copy_tile = [&](const TileRegs& from, TileRegs& to) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        to.k[i][j] = from.k[i][j];
        to.v[i][j] = from.v[i][j];
      }
      to.valid[i] = from.valid[i];
      to.live[i] = from.live[i];
      to.row[i] = from.row[i];
    }
  };
  TileRegs ra, rb;
  BlockIds ba, bb;
  if (spec_hit) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {  // the first tile lies inside the split and before the current token
      ba.blk[i] = spec_blk[i];
      ba.ok[i] = true;
    }
  } else {
    resolve_blocks(0, ba, wave);
  }
  if constexpr (SRC == kSrcPaged) {
    // The static share in wave units: unit u is slot u mod 8 of tile u / 8
    // (the rows a wave covers in one tile).  Each wave starts with its own slot
    // of the first two tiles and then takes the next unit from a workgroup
    // counter in LDS, so a wave whose loads return late takes fewer units and
    // the waves of a workgroup finish closer together (at 128K, FP8: the last
    // wave of a workgroup about 3 us after the first instead of 5; the Full
    // launch 1 us shorter).  An LDS atomic does not wait on the wave's global
    // loads.  Units are claimed two ahead of their loads
    // and their block ids looked up one half-iteration ahead, as in the tile
    // loop; the loads stay unconditional.
    __shared__ int32_t s_unit;
    if (threadIdx.x == 0) s_unit = 2 * kWavesPerGroup;
    __syncthreads();
    const int32_t n_units = n_tiles * kWavesPerGroup;
    auto claim_unit = [&]() {
      int32_t v = 0;
      if (lane == 0) v = atomicAdd(&s_unit, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    auto resolve_unit = [&](int32_t u, BlockIds& B) {
      resolve_blocks(u / kWavesPerGroup, B, u % kWavesPerGroup);
    };
    auto load_unit = [&](int32_t u, const BlockIds& B, TileRegs& R) {
      load_tile(u / kWavesPerGroup, B, R, u % kWavesPerGroup);
    };
    int32_t ub = kWavesPerGroup + wave;
    resolve_unit(ub, bb);
    load_tile(0, ba, ra, wave);
    int32_t uc = claim_unit();
    if (wave < n_units) {
      // ra holds a loaded unit, bb the block ids of unit ub, uc is claimed.
      for (;;) {
        if (ub >= n_units) break;
        resolve_unit(uc, ba);
        load_unit(ub, bb, rb);
        process_tile(ra);
        const int32_t ud = claim_unit();
        if (uc >= n_units) {
          copy_tile(rb, ra);
          break;
        }
        resolve_unit(ud, bb);
        load_unit(uc, ba, ra);
        process_tile(rb);
        ub = ud;
        uc = claim_unit();
      }
      process_tile(ra);
    }
  } else {
  resolve_blocks(1, bb, wave);
  load_tile(0, ba, ra, wave);
  if constexpr (SRC == kSrcRing) {
    if (P.gate_mode == kGateAll) committed = P.seq_len[b];
    if (committed < 0) return;
    ODA_PHASE(1);
    t = committed + 1;
    rst = ring_state(t, P.rows.sink, P.rows.window);
  }
  for (int32_t tile = 0; tile < n_tiles; tile += 2) {
    const bool has_b = tile + 1 < n_tiles;
    resolve_blocks(tile + 2, ba, wave);
    if (has_b) load_tile(tile + 1, bb, rb, wave);
    process_tile(ra);
    if (tile == 0) ODA_PHASE(2);
    resolve_blocks(tile + 3, bb, wave);
    if (tile + 2 < n_tiles) load_tile(tile + 2, ba, ra, wave);
    if (has_b) process_tile(rb);
  }
  }
  ODA_PHASE(3);
  if (n_static < n_all) {
    // Tail pool.  Tile c covers rows n_static + c * TILE .. (the last one ends
    // at n_all).  One round trip claims the workgroup's first two tiles and
    // stages the block ids of every pool row in LDS; after that each claim is
    // issued before the loads of the tile already claimed, so that its result
    // is waited for together with the tile being reduced and two tiles stay
    // in flight.  Pool loads are unconditional (rows outside the tile read
    // the current token's row and are masked when the tile is reduced), which
    // keeps the wait counts exact.
    __shared__ int32_t s_claim[2];
    __shared__ int32_t s_pool_blk[kPoolBlkMax];
    // (uniform per workgroup; readfirstlane makes the loop's exits scalar branches)
    const int32_t pool_tiles = __builtin_amdgcn_readfirstlane((n_all - n_static + TILE - 1) / TILE);
    int32_t* claim = P.claims + ((int64_t)b * P.Hkv + g) * kCounterStride;
    // rows n_static .. n_rows - 1 are positions n_static + 1 .. n_rows
    const int32_t first_blk = n_static >> P.block_shift;
    const int32_t n_blk = n_rows > n_static ? min(((n_rows - 1) >> P.block_shift) - first_blk + 1, kPoolBlkMax) : 0;
    {
      int32_t first = 0;
      if (threadIdx.x == 0) first = __hip_atomic_fetch_add(claim, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      constexpr int IDS = kPoolBlkMax / kGroupThreads;
      int32_t ids[IDS];
#pragma unroll
      for (int k = 0; k < IDS; ++k) {
        const int32_t idx = threadIdx.x + k * kGroupThreads;
        ids[k] = idx < n_blk ? btab[first_blk + idx] : -1;
      }
#pragma unroll
      for (int k = 0; k < IDS; ++k) s_pool_blk[threadIdx.x + k * kGroupThreads] = ids[k];
      if (threadIdx.x == 0) s_claim[0] = first;
      __syncthreads();
    }
    auto resolve_pool = [&](int32_t c, BlockIds& B) {
      const int32_t r0 = n_static + c * TILE;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int32_t row = r0 + (i * kWavesPerGroup + wave) * RPP + rrow;
        const int32_t k = (row >> P.block_shift) - first_blk;
        B.blk[i] = row < n_rows && k < n_blk ? s_pool_blk[k] : -1;
      }
    };
    auto load_pool = [&](int32_t c, const BlockIds& B, TileRegs& R) {
      const int32_t r0 = n_static + c * TILE;
      const int32_t r1 = min(r0 + TILE, n_all);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int32_t pass0 = r0 + (i * kWavesPerGroup + wave) * RPP;
        const int32_t row = pass0 + rrow;
        R.row[i] = row;
        R.live[i] = pass0 < r1;
        const int32_t blk = B.blk[i];
        const bool paged = row < r1 && row < n_rows;
        const bool blk_ok = blk >= 0 && (int64_t)blk < P.num_blocks;
        bad_blk |= paged && !blk_ok;
        const bool from_cache = paged && blk_ok;
        R.valid[i] = from_cache || row == n_rows;
        const char* kb = from_cache ? kbase : static_cast<const char*>(P.k_cur);
        const char* vb = from_cache ? vbase : static_cast<const char*>(P.v_cur);
        const int64_t off =
            from_cache ? ((((int64_t)g * P.num_blocks + blk) << P.block_shift) + (row & bmask)) * D * ES : cur_off;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          constexpr bool kStream = LPR * 16 >= 128;
          R.k[i][j] = kv_load<kStream>(kb + off + (j * LPR + sub) * 16);
          R.v[i][j] = kv_load<kStream>(vb + off + (j * LPR + sub) * 16);
        }
      }
    };
    // (claims are read from LDS: readfirstlane keeps them, and the branches on
    // them, scalar)
    const int32_t c0 = __builtin_amdgcn_readfirstlane(s_claim[0]);
    int32_t c1 = c0 + 1;
    int slot = 1;
    if (c0 < pool_tiles) {
      resolve_pool(c0, ba);
      load_pool(c0, ba, ra);
      // ra holds tile c0 (in flight); c1 is claimed.  Each half of the loop
      // claims the tile after next, loads the claimed one and reduces the
      // one in flight.  The last tile is reduced from ra after the loop (one
      // copy of the reduction on the way out keeps the register count down).
      for (;;) {
        if (c1 >= pool_tiles) break;
        // v is set and read by thread 0 only: left unset elsewhere, it needs
        // no copy where the branch rejoins (a copy would wait for the atomic,
        // and with it for every load issued before it).  The claim is an
        // increment (inc with no wrap bound) rather than an add, which the
        // compiler would rewrite into a wave-wide add whose result it reads
        // back at once.
        int32_t v;
        if (threadIdx.x == 0) v = claim_next(claim);
        resolve_pool(c1, bb);
        load_pool(c1, bb, rb);
        process_tile(ra);
        // Two claim slots: a slot is written again only after the barrier
        // that follows the other slot's write, which every wave reaches after
        // reading this one.
        if (threadIdx.x == 0) s_claim[slot] = v;
        __syncthreads();
        const int32_t c2 = __builtin_amdgcn_readfirstlane(s_claim[slot]);
        slot ^= 1;
        if (c2 >= pool_tiles) {
          copy_tile(rb, ra);
          break;
        }
        if (threadIdx.x == 0) v = claim_next(claim);
        resolve_pool(c2, ba);
        load_pool(c2, ba, ra);
        process_tile(rb);
        if (threadIdx.x == 0) s_claim[slot] = v;
        __syncthreads();
        c1 = __builtin_amdgcn_readfirstlane(s_claim[slot]);
        slot ^= 1;
      }
      process_tile(ra);
    }
  }
  if constexpr (SRC == kSrcPaged)
    if (bad_blk) atomicOr(P.err, (uint32_t)ODA_DEVERR_BLOCK_ID);

  ODA_PHASE(4);
  if constexpr (WITHHOLD) {  // leaves without storing: the merging workgroup waits in vain
    if (split == withheld && !(P.merge_mode == kMergePoll && split + 1 == used)) return;
  }
  constexpr int FOLD_ROWS = kWavesPerGroup;  // rows of the LDS fold: one per wave
  __shared__ float s_wmax[kWavesPerGroup][G];
  constexpr int RS = G * D + 4;  // LDS row stride (words)
  __shared__ float s_o[FOLD_ROWS][RS];
  __shared__ float s_l[kWavesPerGroup][G];
  __shared__ int32_t s_last;
  // Poll mode (the host uses it when every workgroup of the launch is resident
  // at once): the highest split merges and keeps its own partial in LDS; the
  // others store theirs and leave.  Ticket mode: every split stores its
  // partial and the last to take a ticket merges.
  const bool poll = P.merge_mode == kMergePoll;
  const bool merges_here = poll && split + 1 == used;
  __shared__ float s_own_o[G * D];
  __shared__ float s_own_ml[G][2];
  // This workgroup's partial: output element e of head h, or (m, l) of head h.
  auto emit_o = [&](int h, int e, float v) {
    const int64_t row = ((int64_t)b * P.Hq + (int64_t)g * G + h) * P.splits + split;
    if (merges_here)
      s_own_o[h * D + e] = v;
    else
      publish(P.part_o + row * D + e, v);
  };
  auto emit_ml = [&](int h, float mh, float lsum) {
    const int64_t row = ((int64_t)b * P.Hq + (int64_t)g * G + h) * P.splits + split;
    if (merges_here) {
      s_own_ml[h][0] = mh;
      s_own_ml[h][1] = lsum;
    } else {
#pragma unroll
      for (int c = 0; c < D / kWave; ++c) {  // one copy per merging wave
        publish(P.part_ml + (row * (D / kWave) + c) * 2 + 0, mh);
        publish(P.part_ml + (row * (D / kWave) + c) * 2 + 1, lsum);
      }
    }
  };
  // TPO adjacent threads share an output and add FOLD_ROWS / TPO rows each.
  constexpr int TPO = G * D >= kGroupThreads ? 1 : (kGroupThreads / (G * D) >= 4 ? 4 : kGroupThreads / (G * D));
  static_assert(TPO == 1 || TPO == 2 || TPO == 4, "threads per output");

  {
    // Epilogue (one barrier): each wave rescales its row groups onto the
    // wave's maximum per head, adds them (row swaps across the 16-lane rows,
    // then DPP inside them) and stores one LDS row with its (m, l); the fold
    // weighs the 8 wave rows by 2^(m_w - M).
    if constexpr (Gm::MF) {
      // A wave's O^T tiles already sum its rows (its reference is one per
      // head): lane l stores elements 16 mi + 4 (l / 16) .. + 3 of head l % 16;
      // the four lanes of a head add their weight sums.
      const float lw = quarters_sum(l_mf);
      const int h = lane % 16;
      if (h < G) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          *reinterpret_cast<float4*>(&s_o[wave][h * D + 16 * mi + (lane >> 4) * 4]) =
              make_float4(acc_mf[mi][0], acc_mf[mi][1], acc_mf[mi][2], acc_mf[mi][3]);
        if (lane < 16) {
          s_wmax[wave][h] = m_mf;
          s_l[wave][h] = lw;
        }
      }
    } else {
    constexpr int V = G * EPL;
    float v[V];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int mr = __float_as_int(row_group_max<LPR>(m_run[h]));
      const float mw = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(mr, 0)),
                                   __int_as_float(__builtin_amdgcn_readlane(mr, 16))),
                             fmaxf(__int_as_float(__builtin_amdgcn_readlane(mr, 32)),
                                   __int_as_float(__builtin_amdgcn_readlane(mr, 48))));
      const float sc = m_run[h] == -INFINITY ? 0.f : fast_exp2(m_run[h] - mw);
      {
#pragma clang fp contract(off)  // keep the scaling separate so each DPP move folds into an add
        l_acc[h] = row_group_sum<LPR>(l_acc[h] * sc);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[h * EPL + e] = o[h][e] * sc;
      const int li = __float_as_int(l_acc[h]);
      const float lw = (__int_as_float(__builtin_amdgcn_readlane(li, 0)) + __int_as_float(__builtin_amdgcn_readlane(li, 16))) +
                       (__int_as_float(__builtin_amdgcn_readlane(li, 32)) + __int_as_float(__builtin_amdgcn_readlane(li, 48)));
      if (lane == 0) {
        s_wmax[wave][h] = mw;
        s_l[wave][h] = lw;
      }
    }
    // The row swaps first (they leave a quarter of the values per lane), then
    // the row-group sums inside each 16-lane row on what is left.
    float u[V / 4];
    wave_rows_sum_spread<V>(v, u);
#pragma unroll
    for (int k = 0; k < V / 4; ++k) u[k] = row_group_sum<LPR>(u[k]);
    // Lane quarter q holds values q*V/4 .. of its column (value h*EPL + e is
    // element (e / EPV * LPR + col) * EPV + e % EPV of head h): runs of RUN
    // elements, contiguous in the output row.  With LPR < 16 the lanes of a
    // 16-lane row past the first LPR hold copies.
    constexpr int RUN = V / 4 < EPV ? V / 4 : EPV;
    const int q = lane >> 4, col = lane & 15;
    if (col < LPR) {
#pragma unroll
      for (int k0 = 0; k0 < V / 4; k0 += RUN) {
        const int kk = q * (V / 4) + k0;
        const int e = kk % EPL;
        float* dst = &s_o[wave][(kk / EPL) * D + ((e / EPV) * LPR + col) * EPV + e % EPV];
        if constexpr (RUN % 4 == 0) {
#pragma unroll
          for (int k = 0; k < RUN; k += 4)
            *reinterpret_cast<float4*>(dst + k) = make_float4(u[k0 + k], u[k0 + k + 1], u[k0 + k + 2], u[k0 + k + 3]);
        } else {
#pragma unroll
          for (int k = 0; k < RUN; ++k) dst[k] = u[k0 + k];
        }
      }
    }
    }
    __syncthreads();
    ODA_PHASE(5);
    for (int idx = threadIdx.x; idx < G * D * TPO; idx += kGroupThreads) {
      const int out_i = idx / TPO, part = idx % TPO;
      const int h = out_i / D, e = out_i % D;
      float Mh = s_wmax[0][h];
#pragma unroll
      for (int w = 1; w < kWavesPerGroup; ++w) Mh = fmaxf(Mh, s_wmax[w][h]);
      float acc = 0.f, lsum = 0.f;  // every thread also adds its rows' l
#pragma unroll
      for (int r = 0; r < FOLD_ROWS / TPO; ++r) {
        const int row = part * (FOLD_ROWS / TPO) + r;
        const float mw = s_wmax[row][h];
        const float wgt = mw == -INFINITY ? 0.f : fast_exp2(mw - Mh);
        acc = fmaf(wgt, s_o[row][out_i], acc);
        lsum = fmaf(wgt, s_l[row][h], lsum);
      }
      if constexpr (TPO >= 2) {
        acc += xor_lane<1>(acc);
        lsum += xor_lane<1>(lsum);
      }
      if constexpr (TPO >= 4) {
        acc += xor_lane<2>(acc);
        lsum += xor_lane<2>(lsum);
      }
      if (part != 0) continue;
      emit_o(h, e, acc);
      if (e == 0) emit_ml(h, Mh, lsum);
    }
  }

  if (poll) {
    if (!merges_here) {
      ODA_PHASE_STORED(6);
      return;
    }
    __syncthreads();
    ODA_PHASE(6);
    merge_and_write<DT, D, G>(P, b, g, used - 1, true, s_own_o, &s_own_ml[0][0], spin_limit);
    ODA_PHASE_STORED(7);
    // every split has published, so none claims pool tiles any more
    if (threadIdx.x == 0 && n_static < n_all)
      __hip_atomic_store(P.claims + ((int64_t)b * P.Hkv + g) * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // Ticket mode: every wave waits until its device-scope partial stores have
  // completed, then one thread takes a ticket; the holder of the last ticket
  // reads all partials.
  const int64_t pair = (int64_t)b * P.Hkv + g;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  ODA_PHASE(6);
  if (threadIdx.x == 0) {
    const int32_t prev = __hip_atomic_fetch_add(&P.tickets[pair], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == used - 1;
  }
  __syncthreads();
  if (!s_last) return;
  merge_and_write<DT, D, G>(P, b, g, used, false, nullptr, nullptr);
  ODA_PHASE_STORED(7);
  if (threadIdx.x == 0) {  // every ticket (and pool tile) of this launch is taken: ready for the next launch
    __hip_atomic_store(&P.tickets[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n_static < n_all) __hip_atomic_store(P.claims + pair * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int DT, int D, int G, int SRC, bool BALLOT, bool SKIP>
__global__ __launch_bounds__(kGroupThreads) void attention_kernel(AttnParams P) {
  attention_pass<DT, D, G, SRC, BALLOT, SKIP>(P);
}

template <int DT, int D, int G>
__global__ __launch_bounds__(kGroupThreads) void merge_wait_test_kernel(AttnParams P, int32_t withheld,
                                                                        int32_t spin_limit) {
  attention_pass<DT, D, G, kSrcRing, false, true, true>(P, withheld, spin_limit);
}

// ----------------------------------------------------------------------------
// the Full section of a decode step in one launch

// Every workgroup of the launch waits here until all have arrived (the launch
// must fit the chip at once; the host checks).  Thread 0 reads the generation
// before arriving, so the last arrival's bump cannot be missed; the last
// arrival clears the count before the bump, so the next barrier starts from
// zero.  A wait that exceeds the spin limit marks the launch broken
// (ODA_DEVERR_MERGE_WAIT) and every workgroup leaves.
constexpr int32_t kBarrierSpinLimit = 1 << 20;
__device__ __forceinline__ bool grid_barrier(const RegionParams& R) {
  // Every wave's device-scope stores of the layer (partials, the empty marks
  // of its merge, counter resets) have completed before the arrival.  The
  // only data another workgroup reads after the barrier is read with
  // device-scope loads, so no cache-wide fence is needed (one per wave and
  // layer costs tens of microseconds).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ int32_t s_ok;
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(R.bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t arrived = __hip_atomic_fetch_add(R.bar_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int32_t ok = 1;
    if (arrived + 1 == R.groups) {
      __hip_atomic_store(R.bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clear lands before the release of the others
      __hip_atomic_fetch_add(R.bar_gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      for (int32_t spin = 0;; ++spin) {
        // relaxed polls (an acquire load would invalidate the L2 on every poll)
        if (__hip_atomic_load(R.bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gen) break;
        if (__hip_atomic_load(R.bar_broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          ok = 0;
          break;
        }
        if (spin == kBarrierSpinLimit) {
          __hip_atomic_store(R.bar_broken, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          atomicOr(R.err, (uint32_t)ODA_DEVERR_MERGE_WAIT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// The Full pass of every layer of a step (all layers gated, one round of
// workgroups): when the gate fired no request the whole grid leaves at once,
// in place of one empty launch per layer; otherwise the layers run in order,
// each after the previous one's merge, as separate launches would run them.
// P describes layer 0; layer l's cache, queries, current token and outputs
// sit l strides further.
template <int DT, int D, int G>
__global__ __launch_bounds__(kGroupThreads) void full_section_kernel(AttnParams P, RegionParams R) {
  if (*P.call_count <= 0) return;
  for (int32_t l = 0; l < R.layers; ++l) {
    AttnParams Pl = P;
    Pl.k_base = static_cast<const char*>(P.k_base) + l * R.cache_layer_bytes;
    Pl.v_base = static_cast<const char*>(P.v_base) + l * R.cache_layer_bytes;
    Pl.q = static_cast<const char*>(P.q) + l * R.q_layer_bytes;
    Pl.k_cur = static_cast<const char*>(P.k_cur) + l * R.kv_layer_bytes;
    Pl.v_cur = static_cast<const char*>(P.v_cur) + l * R.kv_layer_bytes;
    Pl.out = P.out + l * R.o_layer;
    Pl.lse = P.lse != nullptr ? P.lse + l * R.l_layer : nullptr;
    attention_pass<DT, D, G, kSrcPaged, false, true>(Pl);
    if (l + 1 < R.layers && !grid_barrier(R)) return;
  }
}

// ----------------------------------------------------------------------------
// gate: compaction of the fired requests + accounting

struct GateParams {
  int32_t batch, L, Hq, Hkv, D, esize, sink, window, sw_window, focus;
  int32_t n_gated, n_sliding;
  int64_t recall_flops;
  const float* score;
  float theta;
  const int32_t* seq_len;
  const int64_t* focus_range;
  int32_t* call_list;
  int32_t* call_count;
  int32_t* disp_list;  // optional: the fired requests in dispatch order (longest first)
  int32_t* disp_len;   // their committed lengths, in the same order
  int64_t* full_calls;
  int64_t* counters;
};

// Size of S^L_t U [a,b) (closed form over the merged intervals, plus t).
__device__ int64_t focus_set_size(int32_t t, int32_t s, int32_t w, int64_t fa, int64_t fb) {
  RowSpec rs{};
  rs.source = kSrcPaged;
  rs.focus = 1;
  rs.sink = s;
  rs.window = w;
  return (int64_t)paged_intervals(rs, t, fa, fb).total + 1;
}

// Fired requests up to this many are put in dispatch order by length (more
// keep the list's order).
constexpr int32_t kSortMax = 1024;

__global__ __launch_bounds__(1024) void gate_kernel(GateParams P) {
  __shared__ int32_t s_wave_count[1024 / kWave];
  __shared__ int32_t s_base;
  __shared__ int32_t s_fid[ODA_MAX_BATCH], s_flen[ODA_MAX_BATCH];  // fired requests by list position
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  for (int32_t start = 0; start < P.batch; start += blockDim.x) {
    const int32_t b = start + threadIdx.x;
    bool fire = false;
    int32_t t = 0;
    if (b < P.batch) {
      const int32_t committed = P.seq_len[b];
      t = committed + 1;
      fire = committed >= 0 && P.score[b] > P.theta;  // NaN compares false
      if (committed >= 0) {
        if (P.full_calls) P.full_calls[b] += fire ? 1 : 0;
        if (P.counters) {
          const int64_t per_pos = 4LL * P.Hq * P.D;
          const int64_t bytes_pos = (int64_t)P.Hkv * P.D * 2 * P.esize;
          const int64_t nl_g = min(t, P.sink + P.window);
          int64_t nf_g = t;
          if (P.focus) nf_g = focus_set_size(t, P.sink, P.window, P.focus_range[2 * b], P.focus_range[2 * b + 1]);
          const int64_t n_sw = P.n_sliding > 0 ? min(t, P.sw_window) : 0;
          const int64_t nl = P.n_gated * nl_g + P.n_sliding * n_sw;
          const int64_t nf = P.n_gated * nf_g + P.n_sliding * n_sw;
          const int64_t f_local = per_pos * nl, f_full = per_pos * nf;
          int64_t* c = P.counters + (int64_t)b * ODA_ACCT_N;
          c[ODA_ACCT_STEPS] += 1;
          c[ODA_ACCT_FULL_CALLS] += fire ? 1 : 0;
          c[ODA_ACCT_F_LOCAL] += f_local;
          c[ODA_ACCT_F_FULL_TAKEN] += fire ? f_full : 0;
          c[ODA_ACCT_F_FULL_ALWAYS] += f_full;
          c[ODA_ACCT_DELTA_F] += (fire ? 0 : f_full) - f_local - P.recall_flops;
          c[ODA_ACCT_KV_BYTES] += bytes_pos * (nl + (fire ? nf : 0));
          c[ODA_ACCT_F_RECALL] += P.recall_flops;
        }
      }
    }
    const uint64_t ballot = __ballot(fire);
    if (lane == 0) s_wave_count[wave] = __popcll(ballot);
    __syncthreads();
    int32_t before = s_base;
    for (int w = 0; w < wave; ++w) before += s_wave_count[w];
    const uint64_t lower = lane == 0 ? 0ull : (ballot & ((1ull << lane) - 1ull));
    const int32_t at = before + __popcll(lower);
    if (fire && P.call_list) P.call_list[at] = b;
    if (fire) {
      s_fid[at] = b;
      s_flen[at] = t - 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int32_t total = 0;
      for (int w = 0; w < nwaves; ++w) total += s_wave_count[w];
      s_base += total;
    }
    __syncthreads();
  }
  const int32_t count = s_base;
  if (P.call_list)
    for (int32_t i = count + threadIdx.x; i < P.batch; i += blockDim.x) P.call_list[i] = -1;
  if (threadIdx.x == 0 && P.call_count) *P.call_count = count;
  // Dispatch order of the Full passes: the longest request first (ties by
  // request id), so that when one launch takes several rounds of workgroups
  // the last to be dispatched are the shortest.  Slot i of the list goes to
  // rank i's place: the number of fired requests that come before it.
  if (P.disp_list == nullptr) return;
  if (count > kSortMax) {
    for (int32_t i = threadIdx.x; i < count; i += blockDim.x) {
      P.disp_list[i] = s_fid[i];
      P.disp_len[i] = s_flen[i];
    }
    return;
  }
  for (int32_t i = threadIdx.x; i < count; i += blockDim.x) {
    const int32_t li = s_flen[i];
    int32_t rank = 0;
    for (int32_t j = 0; j < count; ++j) {
      const int32_t lj = s_flen[j];
      rank += (lj > li) || (lj == li && j < i);
    }
    P.disp_list[rank] = s_fid[i];
    P.disp_len[rank] = li;
  }
}

// ----------------------------------------------------------------------------
// fused cross-layer commit

struct CommitParams {
  int32_t L, Hkv, D, esize, sink, window, ring_slots, sw_window, block_shift, max_blocks;
  int32_t batch, ring_batch;
  int64_t num_blocks;
  int32_t n_layers_gated, n_layers_sliding;
  uint8_t kind[ODA_MAX_LAYERS];
  int16_t kidx[ODA_MAX_LAYERS];
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* k_ring;
  void* v_ring;
  void* k_swring;
  void* v_swring;
  int32_t* ring_pos;
  int32_t* swring_pos;
  const int32_t* block_table;
  int32_t* seq_len;
  int32_t* tickets;  // [batch], zero between launches
  uint32_t* err;
};

// grid (layer, request): each workgroup writes one layer of one request; the
// last workgroup of a request (ticket) records t in the ring-slot table and
// advances seq_len, after every workgroup of that request has read it.
__global__ __launch_bounds__(256) void commit_kernel(CommitParams P) {
  const int32_t l = blockIdx.x;
  const int32_t b = blockIdx.y;
  const int32_t committed = P.seq_len[b];
  if (committed < 0) return;
  const int32_t t = committed + 1;
  const int64_t cap = (int64_t)P.max_blocks << P.block_shift;
  const bool has_gated = P.n_layers_gated > 0;
  // The checks below give the same answer in every workgroup of request b, so
  // either all of them take a ticket or none does.
  if (has_gated && t > cap) {
    if (threadIdx.x == 0 && l == 0) atomicOr(P.err, (uint32_t)ODA_DEVERR_CAPACITY);
    return;
  }
  int32_t blk = 0;
  if (has_gated) {
    blk = P.block_table[(int64_t)b * P.max_blocks + ((t - 1) >> P.block_shift)];
    if (blk < 0 || (int64_t)blk >= P.num_blocks) {
      if (threadIdx.x == 0 && l == 0) atomicOr(P.err, (uint32_t)ODA_DEVERR_BLOCK_ID);
      return;
    }
  }
  const int32_t in_blk = (t - 1) & ((1 << P.block_shift) - 1);
  const int32_t gslot = t <= P.sink ? t - 1 : P.sink + (t - P.sink - 1) % P.window;
  const int32_t sslot = P.sw_window > 0 ? (t - 1) % P.sw_window : 0;
  const int64_t row_bytes = (int64_t)P.D * P.esize;
  const int32_t vecs = (int32_t)(row_bytes / 16);
  const int64_t rank = P.kidx[l];
  const bool gated = P.kind[l] == ODA_LAYER_GATED;
  for (int32_t idx = threadIdx.x; idx < P.Hkv * vecs; idx += blockDim.x) {
    const int32_t h = idx / vecs, vi = idx % vecs;
    const int64_t src = (((int64_t)l * P.batch + b) * P.Hkv + h) * row_bytes + vi * 16;
    const uint4 kx = *reinterpret_cast<const uint4*>(static_cast<const char*>(P.k_new) + src);
    const uint4 vx = *reinterpret_cast<const uint4*>(static_cast<const char*>(P.v_new) + src);
    if (gated) {
      const int64_t coff = ((((rank * P.Hkv + h) * P.num_blocks + blk) << P.block_shift) + in_blk) * row_bytes + vi * 16;
      *reinterpret_cast<uint4*>(static_cast<char*>(P.k_cache) + coff) = kx;
      *reinterpret_cast<uint4*>(static_cast<char*>(P.v_cache) + coff) = vx;
      const int64_t roff = (((rank * P.ring_batch + b) * P.Hkv + h) * P.ring_slots + gslot) * row_bytes + vi * 16;
      *reinterpret_cast<uint4*>(static_cast<char*>(P.k_ring) + roff) = kx;
      *reinterpret_cast<uint4*>(static_cast<char*>(P.v_ring) + roff) = vx;
    } else {
      const int64_t roff = (((rank * P.ring_batch + b) * P.Hkv + h) * P.sw_window + sslot) * row_bytes + vi * 16;
      *reinterpret_cast<uint4*>(static_cast<char*>(P.k_swring) + roff) = kx;
      *reinterpret_cast<uint4*>(static_cast<char*>(P.v_swring) + roff) = vx;
    }
  }
  __shared__ int32_t s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t prev = __hip_atomic_fetch_add(&P.tickets[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == P.L - 1;
  }
  __syncthreads();
  if (s_last && threadIdx.x == 0) {
    if (has_gated) P.ring_pos[(int64_t)b * P.ring_slots + gslot] = t;
    if (P.n_layers_sliding > 0) P.swring_pos[(int64_t)b * P.sw_window + sslot] = t;
    P.seq_len[b] = t;
    __hip_atomic_store(&P.tickets[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ----------------------------------------------------------------------------
// prefill of one layer from a dense source, and ring rebuild from the cache

struct PrefillParams {
  int32_t Hkv, D, esize, gated, sink, window, slots, block_shift, max_blocks;
  int64_t num_blocks, src_rows;
  int32_t rank;      // layer rank among its kind
  int32_t ring_batch;  // request stride of rings (max_batch)
  const void* k_src;
  const void* v_src;
  void* k_cache;
  void* v_cache;
  void* k_ring;
  void* v_ring;
  int32_t* ring_pos;
  const int32_t* block_table;
  const int32_t* seq_len;
  uint32_t* err;
  int32_t from_cache;  // ring rebuild: read rows from the paged cache instead of src
};

// grid (x: row chunks, y: request); rows of the paged cache then ring slots
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams P) {
  const int32_t b = blockIdx.y;
  const int32_t committed = P.seq_len[b];
  if (committed < 0) return;
  const int64_t row_bytes = (int64_t)P.D * P.esize;
  const int32_t vecs = (int32_t)(row_bytes / 16);
  const int64_t cap = (int64_t)P.max_blocks << P.block_shift;
  const int32_t bmask = (1 << P.block_shift) - 1;
  if (P.gated && committed > cap) {
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(P.err, (uint32_t)ODA_DEVERR_CAPACITY);
    return;
  }
  if (!P.from_cache && committed > P.src_rows) {
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(P.err, (uint32_t)ODA_DEVERR_CAPACITY);
    return;
  }
  const int32_t* btab = P.block_table + (int64_t)b * P.max_blocks;
  auto cache_off = [&](int32_t p, int32_t h, int32_t vi, bool& ok) -> int64_t {
    const int32_t r0 = p - 1;
    const int32_t blk = btab[r0 >> P.block_shift];
    ok = blk >= 0 && (int64_t)blk < P.num_blocks;
    return (((((int64_t)P.rank * P.Hkv + h) * P.num_blocks + blk) << P.block_shift) + (r0 & bmask)) * row_bytes + vi * 16;
  };
  auto src_off = [&](int32_t p, int32_t h, int32_t vi) -> int64_t {
    return ((((int64_t)b * P.src_rows + (p - 1)) * P.Hkv + h) * row_bytes) + vi * 16;
  };
  const int64_t per_row = (int64_t)P.Hkv * vecs;
  // 1) paged cache rows 1..committed (gated layers, dense source only)
  if (P.gated && !P.from_cache) {
    const int64_t total = (int64_t)committed * per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
      const int32_t p = (int32_t)(idx / per_row) + 1;
      const int32_t rem = (int32_t)(idx % per_row);
      const int32_t h = rem / vecs, vi = rem % vecs;
      bool ok;
      const int64_t co = cache_off(p, h, vi, ok);
      if (!ok) {
        atomicOr(P.err, (uint32_t)ODA_DEVERR_BLOCK_ID);
        continue;
      }
      const int64_t so = src_off(p, h, vi);
      *reinterpret_cast<uint4*>(static_cast<char*>(P.k_cache) + co) =
          *reinterpret_cast<const uint4*>(static_cast<const char*>(P.k_src) + so);
      *reinterpret_cast<uint4*>(static_cast<char*>(P.v_cache) + co) =
          *reinterpret_cast<const uint4*>(static_cast<const char*>(P.v_src) + so);
    }
  }
  // 2) ring slots: the state a one-by-one commit of 1..committed leaves
  const RingState st = ring_state(committed + 1, P.sink, P.window);
  const int64_t total_slots = (int64_t)P.slots * per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total_slots;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int32_t j = (int32_t)(idx / per_row);
    const int32_t rem = (int32_t)(idx % per_row);
    const int32_t h = rem / vecs, vi = rem % vecs;
    bool in_local;
    const int32_t p = ring_slot_position(st, j, in_local);
    if (h == 0 && vi == 0) P.ring_pos[(int64_t)b * P.slots + j] = p;
    if (p == 0) continue;
    const int64_t ro = ((((int64_t)P.rank * P.ring_batch + b) * P.Hkv + h) * P.slots + j) * row_bytes + vi * 16;
    uint4 kx, vx;
    if (P.from_cache) {
      bool ok;
      const int64_t co = cache_off(p, h, vi, ok);
      if (!ok) {
        atomicOr(P.err, (uint32_t)ODA_DEVERR_BLOCK_ID);
        continue;
      }
      kx = *reinterpret_cast<const uint4*>(static_cast<const char*>(P.k_cache) + co);
      vx = *reinterpret_cast<const uint4*>(static_cast<const char*>(P.v_cache) + co);
    } else {
      const int64_t so = src_off(p, h, vi);
      kx = *reinterpret_cast<const uint4*>(static_cast<const char*>(P.k_src) + so);
      vx = *reinterpret_cast<const uint4*>(static_cast<const char*>(P.v_src) + so);
    }
    *reinterpret_cast<uint4*>(static_cast<char*>(P.k_ring) + ro) = kx;
    *reinterpret_cast<uint4*>(static_cast<char*>(P.v_ring) + ro) = vx;
  }
}

// ----------------------------------------------------------------------------
// access-set export

struct AccessParams {
  RowSpec rows;
  int32_t b, capacity_rows, block_shift, max_blocks;
  const int32_t* seq_len;
  const int64_t* focus_range;
  int32_t* positions;
  int64_t capacity;
  int64_t* count;
  uint32_t* err;
};

__global__ __launch_bounds__(256) void access_set_kernel(AccessParams P) {
  __shared__ int32_t s_count;
  if (threadIdx.x == 0) s_count = 0;
  __syncthreads();
  const int32_t committed = P.seq_len[P.b];
  if (committed >= 0) {
    const int32_t t = committed + 1;
    RingState rst{};
    Intervals iv{};
    int32_t n_rows;
    if (P.rows.source == kSrcRing) {
      rst = ring_state(t, P.rows.sink, P.rows.window);
      n_rows = ring_rows(t, P.rows.ring_slots);
    } else {
      int64_t fa = 0, fb = 0;
      if (P.rows.focus) {
        fa = P.focus_range[2 * P.b];
        fb = P.focus_range[2 * P.b + 1];
      }
      iv = paged_intervals(P.rows, t, fa, fb);
      n_rows = iv.total;
    }
    for (int32_t row = threadIdx.x; row <= n_rows; row += blockDim.x) {
      int32_t p;
      if (row == n_rows) {
        p = t;  // the current token, supplied by the caller's k_cur / v_cur
      } else if (P.rows.source == kSrcRing) {
        bool in_local;
        p = ring_slot_position(rst, row, in_local);
        if (!in_local) p = 0;
      } else {
        p = interval_position(iv, row);
      }
      if (p > 0) {
        const int32_t at = atomicAdd(&s_count, 1);
        if (at < P.capacity) P.positions[at] = p;
        else atomicOr(P.err, (uint32_t)ODA_DEVERR_OUT_CAPACITY);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) *P.count = s_count;
}

// ----------------------------------------------------------------------------
// small helpers

__global__ void fill_kernel(uint32_t* p, int64_t words, uint32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

struct StageParams {
  int32_t n;
  const void* src[8];
  void* dst[8];
  int64_t bytes[8];
  int64_t* counter;  // [0] step index, [1] ticket (zero between launches)
  int64_t num_steps;
};

// Copies step k's inputs (k = counter[0] mod num_steps); the last workgroup to
// finish -- after every workgroup has read k -- advances counter[0].
__global__ __launch_bounds__(256) void stage_kernel(StageParams P) {
  const int64_t k = *P.counter % P.num_steps;
  for (int i = 0; i < P.n; ++i) {
    const int64_t vecs = P.bytes[i] / 16;
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const char*>(P.src[i]) + k * P.bytes[i]);
    uint4* d = reinterpret_cast<uint4*>(P.dst[i]);
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < vecs; v += (int64_t)gridDim.x * blockDim.x)
      d[v] = s[v];
  }
  __shared__ int32_t s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t prev = __hip_atomic_fetch_add(P.counter + 1, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (int64_t)gridDim.x - 1;
  }
  __syncthreads();
  if (s_last && threadIdx.x == 0) {
    P.counter[0] += 1;
    __hip_atomic_store(P.counter + 1, (int64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void advance_kernel(int64_t* counter) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *counter += 1;
}

// ----------------------------------------------------------------------------
// dispatch over the built instantiations

template <int DT, int D, int G>
int launch_attention_t(const AttnParams& a, int32_t batch, oda_stream s) {
  dim3 grid(a.splits, a.Hkv, batch);
  const bool ballot = a.gate_mode == kGateBallot;
  const dim3 block(kGroupThreads);
  if (a.rows.source == kSrcRing) {
    // Splits no longer than a tile (the usual case at small batch) skip empty passes.
    const int32_t units = (a.rows.ring_slots + 1 + kSplitRowUnit - 1) / kSplitRowUnit;
    const bool skip = (int64_t)((units + a.splits - 1) / a.splits) * kSplitRowUnit <= Geo<DT, D, kSrcRing, G>::TILE;
    if (ballot) {
      if (skip) hipLaunchKernelGGL((attention_kernel<DT, D, G, kSrcRing, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((attention_kernel<DT, D, G, kSrcRing, true, false>), grid, block, 0, s, a);
    } else {
      if (skip) hipLaunchKernelGGL((attention_kernel<DT, D, G, kSrcRing, false, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((attention_kernel<DT, D, G, kSrcRing, false, false>), grid, block, 0, s, a);
    }
  } else {
    if (ballot) hipLaunchKernelGGL((attention_kernel<DT, D, G, kSrcPaged, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attention_kernel<DT, D, G, kSrcPaged, false, true>), grid, block, 0, s, a);
  }
  return (int)hipGetLastError();
}

template <int DT, int D, int G>
int launch_full_section_t(const AttnParams& a, const RegionParams& r, int32_t batch, oda_stream s) {
  dim3 grid(a.splits, a.Hkv, batch);
  hipLaunchKernelGGL((full_section_kernel<DT, D, G>), grid, dim3(kGroupThreads), 0, s, a, r);
  return (int)hipGetLastError();
}

// Groups of 8 are built for bf16 and FP8 (both products on MFMA) and for f32
// with d = 64, whose row fits one 16-byte chunk per lane of a 16-lane row with
// eight heads' accumulators (the host reports f32 with d = 128 unsupported).
template <int DT, int D>
constexpr bool kGroup8Built = DT != ODA_F32 || D == 64;

template <int DT, int D>
int launch_attention_d(const Plan& p, const AttnParams& a, int32_t batch, oda_stream s) {
  switch (p.G) {
    case 1: return launch_attention_t<DT, D, 1>(a, batch, s);
    case 2: return launch_attention_t<DT, D, 2>(a, batch, s);
    case 4: return launch_attention_t<DT, D, 4>(a, batch, s);
    case 8:
      if constexpr (kGroup8Built<DT, D>) return launch_attention_t<DT, D, 8>(a, batch, s);
      return (int)hipErrorInvalidValue;
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

// Rows per tile of the kernel built for (dtype, d, source, group): the same
// Geo<> instantiation the launch dispatches to (f32 groups of 8 exist for
// d = 64 only; the host reports the other case unsupported before asking).
template <int SRC, int G>
int tile_rows_src(int32_t dtype, int32_t head_dim) {
  if (dtype == ODA_BF16) return head_dim == 128 ? Geo<ODA_BF16, 128, SRC, G>::TILE : Geo<ODA_BF16, 64, SRC, G>::TILE;
  if (dtype == ODA_FP8_E4M3)
    return head_dim == 128 ? Geo<ODA_FP8_E4M3, 128, SRC, G>::TILE : Geo<ODA_FP8_E4M3, 64, SRC, G>::TILE;
  if constexpr (kGroup8Built<ODA_F32, 128> || G < 8) {
    if (head_dim == 128) return Geo<ODA_F32, 128, SRC, G>::TILE;
  }
  return head_dim == 128 ? 0 : Geo<ODA_F32, 64, SRC, G>::TILE;
}

template <int SRC>
int tile_rows_g(int32_t dtype, int32_t head_dim, int32_t group) {
  switch (group) {
    case 1: return tile_rows_src<SRC, 1>(dtype, head_dim);
    case 2: return tile_rows_src<SRC, 2>(dtype, head_dim);
    case 4: return tile_rows_src<SRC, 4>(dtype, head_dim);
    case 8: return tile_rows_src<SRC, 8>(dtype, head_dim);
    default: return 0;
  }
}

int tile_rows_for(int32_t dtype, int32_t head_dim, int32_t source, int32_t group) {
  return source == kSrcRing ? tile_rows_g<kSrcRing>(dtype, head_dim, group)
                            : tile_rows_g<kSrcPaged>(dtype, head_dim, group);
}

template <int DT, int D>
int launch_full_section_d(const Plan& p, const AttnParams& a, const RegionParams& r, int32_t batch, oda_stream s) {
  switch (p.G) {
    case 1: return launch_full_section_t<DT, D, 1>(a, r, batch, s);
    case 2: return launch_full_section_t<DT, D, 2>(a, r, batch, s);
    case 4: return launch_full_section_t<DT, D, 4>(a, r, batch, s);
    case 8:
      if constexpr (kGroup8Built<DT, D>) return launch_full_section_t<DT, D, 8>(a, r, batch, s);
      return (int)hipErrorInvalidValue;
    default: return (int)hipErrorInvalidValue;
  }
}

int launch_full_section(const Plan& p, const AttnParams& a, const RegionParams& r, int32_t batch, oda_stream s) {
  if (batch <= 0) return 0;
  if (p.dtype == ODA_BF16) {
    if (p.D == 128) return launch_full_section_d<ODA_BF16, 128>(p, a, r, batch, s);
    return launch_full_section_d<ODA_BF16, 64>(p, a, r, batch, s);
  }
  if (p.dtype == ODA_FP8_E4M3) {
    if (p.D == 128) return launch_full_section_d<ODA_FP8_E4M3, 128>(p, a, r, batch, s);
    return launch_full_section_d<ODA_FP8_E4M3, 64>(p, a, r, batch, s);
  }
  if (p.D == 128) return launch_full_section_d<ODA_F32, 128>(p, a, r, batch, s);
  return launch_full_section_d<ODA_F32, 64>(p, a, r, batch, s);
}

int compute_units() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

int launch_attention(const Plan& p, const AttnParams& a, int32_t batch, oda_stream s) {
  if (batch <= 0) return 0;
  if (p.dtype == ODA_BF16) {
    if (p.D == 128) return launch_attention_d<ODA_BF16, 128>(p, a, batch, s);
    return launch_attention_d<ODA_BF16, 64>(p, a, batch, s);
  }
  if (p.dtype == ODA_FP8_E4M3) {
    if (p.D == 128) return launch_attention_d<ODA_FP8_E4M3, 128>(p, a, batch, s);
    return launch_attention_d<ODA_FP8_E4M3, 64>(p, a, batch, s);
  }
  if (p.D == 128) return launch_attention_d<ODA_F32, 128>(p, a, batch, s);
  return launch_attention_d<ODA_F32, 64>(p, a, batch, s);
}

int launch_attention_merge_wait(const Plan& p, const AttnParams& a, int32_t batch, int32_t withheld,
                                int32_t spin_limit, oda_stream s) {
  if (batch <= 0) return 0;
  if (p.dtype != ODA_BF16 || a.rows.source != kSrcRing || (p.G != 1 && p.G != 2)) return (int)hipErrorInvalidValue;
  dim3 grid(a.splits, a.Hkv, batch);
  const dim3 block(kGroupThreads);
  if (p.D == 128) {
    if (p.G == 1) hipLaunchKernelGGL((merge_wait_test_kernel<ODA_BF16, 128, 1>), grid, block, 0, s, a, withheld, spin_limit);
    else hipLaunchKernelGGL((merge_wait_test_kernel<ODA_BF16, 128, 2>), grid, block, 0, s, a, withheld, spin_limit);
  } else {
    if (p.G == 1) hipLaunchKernelGGL((merge_wait_test_kernel<ODA_BF16, 64, 1>), grid, block, 0, s, a, withheld, spin_limit);
    else hipLaunchKernelGGL((merge_wait_test_kernel<ODA_BF16, 64, 2>), grid, block, 0, s, a, withheld, spin_limit);
  }
  return (int)hipGetLastError();
}

int launch_gate(const Plan& p, const oda_kv& kv, int32_t batch, const float* score, float theta,
                int32_t* call_list, int32_t* call_count, int32_t* disp_list, int32_t* disp_len,
                int64_t* full_calls, int64_t* counters, oda_stream s) {
  if (batch <= 0) return 0;
  GateParams g{};
  g.batch = batch;
  g.L = p.L;
  g.Hq = p.Hq;
  g.Hkv = p.Hkv;
  g.D = p.D;
  g.esize = p.esize;
  g.sink = p.sink;
  g.window = p.window;
  g.sw_window = p.sw_window;
  g.focus = p.focus;
  g.n_gated = p.Lg;
  g.n_sliding = p.Ls;
  g.recall_flops = p.recall_flops;
  g.score = score;
  g.theta = theta;
  g.seq_len = kv.seq_len;
  g.focus_range = kv.focus_range;
  g.call_list = call_list;
  g.call_count = call_count;
  g.disp_list = disp_list;
  g.disp_len = disp_len;
  g.full_calls = full_calls;
  g.counters = counters;
  const int threads = batch >= 1024 ? 1024 : ((batch + 63) / 64) * 64;
  hipLaunchKernelGGL(gate_kernel, dim3(1), dim3(threads), 0, s, g);
  return (int)hipGetLastError();
}

int launch_commit(const Plan& p, const oda_kv& kv, int32_t batch, const void* k_new,
                  const void* v_new, int32_t* tickets, uint32_t* err, oda_stream s) {
  if (batch <= 0) return 0;
  CommitParams c{};
  c.L = p.L;
  c.Hkv = p.Hkv;
  c.D = p.D;
  c.esize = p.esize;
  c.sink = p.sink;
  c.window = p.window;
  c.ring_slots = p.ring_slots;
  c.sw_window = p.sw_window;
  c.block_shift = p.block_shift;
  c.max_blocks = p.max_blocks;
  c.batch = batch;           // k_new / v_new are [L][batch][Hkv][d]
  c.ring_batch = p.max_batch;  // rings are [L?][max_batch][Hkv][slots][d]
  c.num_blocks = kv.num_blocks;
  c.n_layers_gated = p.Lg;
  c.n_layers_sliding = p.Ls;
  for (int l = 0; l < p.L; ++l) {
    c.kind[l] = p.kind[l];
    c.kidx[l] = p.kidx[l];
  }
  c.k_new = k_new;
  c.v_new = v_new;
  c.k_cache = kv.k_cache;
  c.v_cache = kv.v_cache;
  c.k_ring = kv.k_ring;
  c.v_ring = kv.v_ring;
  c.k_swring = kv.k_swring;
  c.v_swring = kv.v_swring;
  c.ring_pos = kv.ring_pos;
  c.swring_pos = kv.swring_pos;
  c.block_table = kv.block_table;
  c.seq_len = kv.seq_len;
  c.tickets = tickets;
  c.err = err;
  hipLaunchKernelGGL(commit_kernel, dim3(p.L, batch), dim3(256), 0, s, c);
  return (int)hipGetLastError();
}

int launch_prefill(const Plan& p, const oda_kv& kv, int32_t batch, int32_t layer,
                   const void* k_src, const void* v_src, int64_t src_rows, uint32_t* err,
                   oda_stream s) {
  if (batch <= 0) return 0;
  PrefillParams f{};
  const bool gated = p.kind[layer] == ODA_LAYER_GATED;
  f.Hkv = p.Hkv;
  f.D = p.D;
  f.esize = p.esize;
  f.gated = gated;
  f.sink = gated ? p.sink : 0;
  f.window = gated ? p.window : p.sw_window;
  f.slots = gated ? p.ring_slots : p.sw_window;
  f.block_shift = p.block_shift;
  f.max_blocks = p.max_blocks;
  f.num_blocks = kv.num_blocks;
  f.src_rows = src_rows;
  f.rank = p.kidx[layer];
  f.ring_batch = p.max_batch;
  f.k_src = k_src;
  f.v_src = v_src;
  f.k_cache = kv.k_cache;
  f.v_cache = kv.v_cache;
  f.k_ring = gated ? kv.k_ring : kv.k_swring;
  f.v_ring = gated ? kv.v_ring : kv.v_swring;
  f.ring_pos = gated ? kv.ring_pos : kv.swring_pos;
  f.block_table = kv.block_table;
  f.seq_len = kv.seq_len;
  f.err = err;
  f.from_cache = 0;
  const int64_t per_row = (int64_t)p.Hkv * p.D * p.esize / 16;
  int64_t work = (src_rows > f.slots ? src_rows : f.slots) * per_row;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)blocks, batch), dim3(256), 0, s, f);
  return (int)hipGetLastError();
}

int launch_ring_init(const Plan& p, const oda_kv& kv, int32_t batch, uint32_t* err, oda_stream s) {
  if (batch <= 0) return 0;
  for (int l = 0; l < p.L; ++l) {
    if (p.kind[l] != ODA_LAYER_GATED) continue;
    PrefillParams f{};
    f.Hkv = p.Hkv;
    f.D = p.D;
    f.esize = p.esize;
    f.gated = 1;
    f.sink = p.sink;
    f.window = p.window;
    f.slots = p.ring_slots;
    f.block_shift = p.block_shift;
    f.max_blocks = p.max_blocks;
    f.num_blocks = kv.num_blocks;
    f.src_rows = 0;
    f.rank = p.kidx[l];
    f.ring_batch = p.max_batch;
    f.k_cache = kv.k_cache;
    f.v_cache = kv.v_cache;
    f.k_ring = kv.k_ring;
    f.v_ring = kv.v_ring;
    f.ring_pos = kv.ring_pos;
    f.block_table = kv.block_table;
    f.seq_len = kv.seq_len;
    f.err = err;
    f.from_cache = 1;
    const int64_t work = (int64_t)p.ring_slots * p.Hkv * p.D * p.esize / 16;
    const int64_t blocks = (work + 255) / 256;
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)blocks, batch), dim3(256), 0, s, f);
    const int rc = (int)hipGetLastError();
    if (rc) return rc;
  }
  return 0;
}

int launch_access_set(const Plan& p, const oda_kv& kv, int32_t layer, int32_t b, int32_t mode,
                      int32_t* positions, int64_t capacity, int64_t* count, uint32_t* err,
                      oda_stream s) {
  AccessParams a{};
  const bool gated = p.kind[layer] == ODA_LAYER_GATED;
  a.rows.source = (gated && mode == 1) ? kSrcPaged : kSrcRing;
  a.rows.focus = p.focus;
  a.rows.sink = gated ? p.sink : 0;
  a.rows.window = gated ? p.window : p.sw_window;
  a.rows.ring_slots = gated ? p.ring_slots : p.sw_window;
  a.b = b;
  a.block_shift = p.block_shift;
  a.max_blocks = p.max_blocks;
  a.seq_len = kv.seq_len;
  a.focus_range = kv.focus_range;
  a.positions = positions;
  a.capacity = capacity;
  a.count = count;
  a.err = err;
  hipLaunchKernelGGL(access_set_kernel, dim3(1), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

int launch_fill(void* ptr, size_t bytes, uint32_t value, oda_stream s) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words <= 0) return 0;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(ptr), words, value);
  return (int)hipGetLastError();
}
int launch_clear(void* ptr, size_t bytes, oda_stream s) { return launch_fill(ptr, bytes, 0u, s); }
int launch_workspace_init(void* ws, size_t partials_off, size_t total, oda_stream s) {
  const int e = launch_fill(ws, partials_off, 0u, s);
  if (e != 0) return e;
  return launch_fill(static_cast<char*>(ws) + partials_off, total - partials_off, kPartialEmpty, s);
}

int launch_stage(int32_t n, const void* const* src, void* const* dst, const int64_t* bytes,
                 int64_t* counter, int64_t num_steps, oda_stream s) {
  StageParams sp{};
  sp.n = n;
  int64_t most = 0;
  for (int i = 0; i < n; ++i) {
    sp.src[i] = src[i];
    sp.dst[i] = dst[i];
    sp.bytes[i] = bytes[i];
    if (bytes[i] > most) most = bytes[i];
  }
  sp.counter = counter;
  sp.num_steps = num_steps;
  int64_t blocks = (most / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 256) blocks = 256;
  hipLaunchKernelGGL(stage_kernel, dim3((unsigned)blocks), dim3(256), 0, s, sp);
  return (int)hipGetLastError();
}

int launch_advance(int64_t* counter, oda_stream s) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, counter);
  return (int)hipGetLastError();
}

// ----------------------------------------------------------------------------
// recall head stand-in: q = w2 . max(W1 x + b1, 0) + b2 for every request

constexpr int kRecallRowsPerWave = 2;        // hidden units per wave (one workgroup: 16)
constexpr int kRecallBatchChunk = 8;         // requests whose x sits in LDS at once
constexpr int kRecallLdsBytes = 48 * 1024;   // x chunk: at most this many bytes
constexpr int kRecallVecs = 4;               // 16-byte W1 vectors per lane per row in flight

struct RecallParams {
  int32_t in_dim, hidden, batch, chunk;  // chunk: requests per LDS round (<= kRecallBatchChunk)
  const uint4* w1;
  const float* b1;
  const float* w2;
  float b2;
  const uint4* x;
  float* scores;
  float* partial;   // [groups][batch]
  int32_t* ticket;  // zero between launches
};

// Workgroup g owns hidden units [16 g, 16 g + 16), two per wave.  For each
// chunk of requests the x rows are staged in LDS; every wave streams its two
// W1 rows once per chunk with 16-byte loads (both rows' next four vectors per
// lane in flight together), multiplies them with every staged x row and adds
// w2_j max(u_j, 0) into per-request sums.  The workgroup's sums are published
// device-wide and the last workgroup adds all of them with b2.
__global__ __launch_bounds__(kGroupThreads) void recall_kernel(RecallParams P) {
  extern __shared__ uint4 s_x[];  // [chunk][in_dim / 8]
  __shared__ float s_part[kWavesPerGroup][kRecallBatchChunk];
  __shared__ int32_t s_last;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int32_t vecs = P.in_dim / 8;  // 16-byte vectors per row
  const int32_t row0 = blockIdx.x * (kWavesPerGroup * kRecallRowsPerWave) + wave * kRecallRowsPerWave;
  bool live[kRecallRowsPerWave];
  const uint4* wrow[kRecallRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRecallRowsPerWave; ++r) {
    live[r] = row0 + r < P.hidden;
    wrow[r] = P.w1 + (int64_t)(live[r] ? row0 + r : 0) * vecs;
  }
  for (int32_t c0 = 0; c0 < P.batch; c0 += P.chunk) {
    const int32_t nb = min(P.chunk, P.batch - c0);
    __syncthreads();  // the previous chunk's LDS reads are done
    for (int32_t i = threadIdx.x; i < nb * vecs; i += kGroupThreads)
      s_x[i] = P.x[(int64_t)c0 * vecs + i];
    __syncthreads();
    float acc[kRecallRowsPerWave][kRecallBatchChunk];
#pragma unroll
    for (int r = 0; r < kRecallRowsPerWave; ++r)
#pragma unroll
      for (int b = 0; b < kRecallBatchChunk; ++b) acc[r][b] = 0.f;
    for (int32_t v0 = 0; v0 < vecs; v0 += kWave * kRecallVecs) {
      uint4 w[kRecallRowsPerWave][kRecallVecs];
#pragma unroll
      for (int r = 0; r < kRecallRowsPerWave; ++r)
#pragma unroll
        for (int k = 0; k < kRecallVecs; ++k) {
          const int32_t v = v0 + k * kWave + lane;
          w[r][k] = (live[r] && v < vecs) ? wrow[r][v] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int k = 0; k < kRecallVecs; ++k) {
        const int32_t v = v0 + k * kWave + lane;
        if (v >= vecs) break;
#pragma unroll
        for (int b = 0; b < kRecallBatchChunk; ++b) {
          if (b < nb) {
            const uint4 xv = s_x[b * vecs + v];
#pragma unroll
            for (int r = 0; r < kRecallRowsPerWave; ++r) {
              float a = acc[r][b];
              a = dot2_bf16(w[r][k].x, xv.x, a);
              a = dot2_bf16(w[r][k].y, xv.y, a);
              a = dot2_bf16(w[r][k].z, xv.z, a);
              a = dot2_bf16(w[r][k].w, xv.w, a);
              acc[r][b] = a;
            }
          }
        }
      }
    }
    float sums[kRecallBatchChunk];
#pragma unroll
    for (int b = 0; b < kRecallBatchChunk; ++b) sums[b] = 0.f;
#pragma unroll
    for (int r = 0; r < kRecallRowsPerWave; ++r) {
      if (!live[r]) continue;  // uniform across the wave
      const float b1 = P.b1[row0 + r], w2 = P.w2[row0 + r];
#pragma unroll
      for (int b = 0; b < kRecallBatchChunk; ++b) {
        if (b < nb) {
          const float u = sum_over<1, 32>(acc[r][b]) + b1;
          sums[b] = fmaf(w2, fmaxf(u, 0.f), sums[b]);
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < kRecallBatchChunk; ++b) s_part[wave][b] = sums[b];
    }
    __syncthreads();
    if (threadIdx.x < nb) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kWavesPerGroup; ++w) t += s_part[w][threadIdx.x];
      publish(P.partial + (int64_t)blockIdx.x * P.batch + c0 + threadIdx.x, t);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t prev = __hip_atomic_fetch_add(P.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (int32_t)gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  // One wave per request: every lane loads up to eight partials at once, then
  // the wave adds them.
  const int32_t groups = (int32_t)gridDim.x;
  for (int32_t b = wave; b < P.batch; b += kWavesPerGroup) {
    float t = 0.f;
    for (int32_t g0 = 0; g0 < groups; g0 += 8 * kWave) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int32_t g = g0 + k * kWave + lane;
        v[k] = g < groups ? collect(P.partial + (int64_t)g * P.batch + b) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) t += v[k];
    }
    t = sum_over<1, 32>(t);
    if (lane == 0) P.scores[b] = t + P.b2;
  }
  if (threadIdx.x == 0) __hip_atomic_store(P.ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int recall_groups(int32_t hidden) {
  const int32_t per = kWavesPerGroup * kRecallRowsPerWave;
  return (hidden + per - 1) / per;
}

size_t recall_workspace_bytes(int32_t hidden, int32_t batch) {
  // ticket word, then the partial sums
  return 256 + ((sizeof(float) * (size_t)recall_groups(hidden) * (size_t)batch + 255) & ~(size_t)255);
}

int launch_recall(const oda_recall_head& h, int32_t batch, const void* x, float* scores, void* ws,
                  oda_stream s) {
  if (batch <= 0) return 0;
  RecallParams P{};
  P.in_dim = h.in_dim;
  P.hidden = h.hidden;
  P.batch = batch;
  const int32_t row_bytes = h.in_dim * 2;
  int32_t chunk = kRecallLdsBytes / row_bytes;
  if (chunk > kRecallBatchChunk) chunk = kRecallBatchChunk;
  if (chunk < 1) chunk = 1;
  P.chunk = chunk;
  P.w1 = static_cast<const uint4*>(h.w1);
  P.b1 = h.b1;
  P.w2 = h.w2;
  P.b2 = h.b2;
  P.x = static_cast<const uint4*>(x);
  P.scores = scores;
  P.ticket = static_cast<int32_t*>(ws);
  P.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + 256);
  const size_t lds = (size_t)chunk * row_bytes;
  hipLaunchKernelGGL(recall_kernel, dim3(recall_groups(h.hidden)), dim3(kGroupThreads), lds, s, P);
  return (int)hipGetLastError();
}

// ----------------------------------------------------------------------------
// static scratch of the step entry point that allocates nothing

// The workspace of oda_step_static: one copy per GPU, held from the library's
// load until the process ends.  In host code `scratch` names a host-side
// stand-in, never its device copy: its device address is taken once per
// device with hipGetSymbolAddress (that device current) and only that address
// is used afterwards.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

int static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 1;
  }
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return 2;
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int host_device_pointer(void* host_ptr, void** device_ptr) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, host_ptr) != hipSuccess) {
    (void)hipGetLastError();  // an unknown pointer leaves an error behind: clear it
    return 1;
  }
  if (attr.type != hipMemoryTypeHost) return 1;
  void* dev = nullptr;
  if (hipHostGetDevicePointer(&dev, host_ptr, 0) != hipSuccess || dev == nullptr) {
    (void)hipGetLastError();
    return 2;
  }
  *device_ptr = dev;
  return 0;
}

}  // namespace oda

#ifdef ODA_PHASE_STAMPS
extern "C" int oda_phase_stamps_read(unsigned long long* stamps, unsigned* xcc, size_t groups) {
  if (groups > (size_t)oda::kPhaseGroups || !stamps || !xcc) return (int)hipErrorInvalidValue;
  hipError_t e = hipMemcpyFromSymbol(stamps, HIP_SYMBOL(oda::g_phase_stamps),
                                     groups * oda::kPhases * sizeof(unsigned long long), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return (int)e;
  return (int)hipMemcpyFromSymbol(xcc, HIP_SYMBOL(oda::g_phase_xcc), groups * sizeof(unsigned), 0,
                                  hipMemcpyDeviceToHost);
}

extern "C" int oda_phase_stamps_clear(void) {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(oda::g_phase_stamps));
  if (e != hipSuccess) return (int)e;
  return (int)hipMemset(p, 0, sizeof(unsigned long long) * oda::kPhaseGroups * oda::kPhases);
}
#endif
