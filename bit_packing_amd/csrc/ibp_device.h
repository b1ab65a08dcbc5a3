// ibp_device.h -- device helpers shared by the gfx950 kernels of the IBP codec:
// 64-lane wave primitives, run-decomposed bit extract/deposit, LDS bit fields,
// 16-byte loads and agent-scope atomics.
#pragma once

#include "ibp.h"
#include "ibp_internal.h"

namespace ibp {
namespace dev {

// s_waitcnt immediate (gfx9 encoding) that waits for all vector memory operations
// and nothing else: vmcnt 0 (bits 3:0 and 15:14), expcnt 7 (6:4), lgkmcnt 15 (11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

// ------------------------------------------------------------------ wave helpers

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in the lanes below this one (v_mbcnt).
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc(uint64_t m) { return (uint32_t)__builtin_popcountll(m); }

__device__ __forceinline__ uint64_t low_lanes(uint32_t k) {  // bits [0, k), k <= 64
  return k >= 64 ? ~0ull : ((1ull << k) - 1ull);
}

// readfirstlane returns int: convert through uint32_t so nothing is sign-extended.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | lo;
}

// Orders this wavefront's LDS accesses around the call.  LDS instructions of one
// wavefront execute in program order, so only the compiler needs fencing.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes, in DPP: row shifts by 1, 2, 4 and 8
// within each row of 16 lanes, then the last lane of row 0 (2) broadcast into row
// 1 (3), then lane 31 into rows 2 and 3.  Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_sum32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ------------------------------------------------------------------ bit moves

// Parallel bit extract / deposit over the free (non-Mask) positions, one shift,
// AND and OR per run.  NR = number of runs when known at compile time (1..8),
// NR = 0 for a loop over the runtime count.
template <typename T, uint32_t NR> __device__ __forceinline__ T extract_free(T v, const Runs &rr) {
  T out = 0;
  if constexpr (NR == 0) {
    for (uint32_t r = 0; r < rr.n; ++r) out |= (v >> rr.shift[r]) & (T)rr.pmask[r];
  } else {
#pragma unroll
    for (uint32_t r = 0; r < NR; ++r) out |= (v >> rr.shift[r]) & (T)rr.pmask[r];
  }
  return out;
}

template <typename T, uint32_t NR> __device__ __forceinline__ T deposit_free(T x, const Runs &rr) {
  T out = 0;
  if constexpr (NR == 0) {
    for (uint32_t r = 0; r < rr.n; ++r) out |= (x & (T)rr.pmask[r]) << rr.shift[r];
  } else {
#pragma unroll
    for (uint32_t r = 0; r < NR; ++r) out |= (x & (T)rr.pmask[r]) << rr.shift[r];
  }
  return out;
}

// Bit extract for a per-lane free-position mask F (the lane's own Mask, so runs
// differ between lanes): one step per run, with integer-width operations on U:
// R = F & ~(F + lowest set bit) is F's lowest run of consecutive set positions.
template <typename U> __device__ __forceinline__ uint32_t ctz_u(U v) {
  return sizeof(U) > 4 ? (uint32_t)__builtin_ctzll((uint64_t)v) : (uint32_t)__builtin_ctz((uint32_t)v);
}
template <typename U> __device__ __forceinline__ uint32_t popc_u(U v) {
  return sizeof(U) > 4 ? (uint32_t)__builtin_popcountll((uint64_t)v) : (uint32_t)__builtin_popcount((uint32_t)v);
}

template <typename U> __device__ __forceinline__ U extract_runs(U v, U F) {
  U out = 0;
  uint32_t k = 0;
  while (F) {
    const U R = F & ~(F + (F & (U)(0 - F)));
    out |= ((v & R) >> ctz_u(F)) << k;
    k += popc_u(R);
    F ^= R;
  }
  return out;
}

// ------------------------------------------------------------------ LDS bit fields

__device__ __forceinline__ uint32_t lds_bit(const uint32_t *s, uint32_t q) {
  return (s[q >> 5] >> (q & 31u)) & 1u;
}

// sizeof(T)*8 bits starting at local bit q (stream order, low bit first).
template <typename T> __device__ __forceinline__ T lds_field(const uint32_t *s, uint32_t q);

template <> __device__ __forceinline__ uint16_t lds_field<uint16_t>(const uint32_t *s, uint32_t q) {
  const uint32_t d = q >> 5, sh = q & 31u;
  return (uint16_t)__builtin_amdgcn_alignbit(s[d + 1], s[d], sh);
}

template <> __device__ __forceinline__ uint32_t lds_field<uint32_t>(const uint32_t *s, uint32_t q) {
  const uint32_t d = q >> 5, sh = q & 31u;
  return __builtin_amdgcn_alignbit(s[d + 1], s[d], sh);
}

template <> __device__ __forceinline__ uint64_t lds_field<uint64_t>(const uint32_t *s, uint32_t q) {
  const uint32_t d = q >> 5, sh = q & 31u;
  const uint32_t w0 = s[d], w1 = s[d + 1], w2 = s[d + 2];
  const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, sh);
  const uint32_t hi = __builtin_amdgcn_alignbit(w2, w1, sh);
  return ((uint64_t)hi << 32) | lo;
}

// OR a field whose bits above its length are 0 into LDS at bit q.
__device__ __forceinline__ void lds_or_field(uint32_t *s, uint32_t q, uint32_t x) {
  const uint32_t d = q >> 5, sh = q & 31u;
  const uint32_t lo = x << sh;
  const uint32_t hi = sh ? (x >> (32u - sh)) : 0u;
  if (lo) atomicOr(&s[d], lo);
  if (hi) atomicOr(&s[d + 1], hi);
}

__device__ __forceinline__ void lds_or_field(uint32_t *s, uint32_t q, uint16_t x) { lds_or_field(s, q, (uint32_t)x); }

__device__ __forceinline__ void lds_or_field(uint32_t *s, uint32_t q, uint64_t x) {
  const uint32_t d = q >> 5, sh = q & 31u;
  const uint32_t x0 = (uint32_t)x, x1 = (uint32_t)(x >> 32);
  const uint32_t w0 = x0 << sh;
  const uint32_t w1 = sh ? ((x1 << sh) | (x0 >> (32u - sh))) : x1;
  const uint32_t w2 = sh ? (x1 >> (32u - sh)) : 0u;
  if (w0) atomicOr(&s[d], w0);
  if (w1) atomicOr(&s[d + 1], w1);
  if (w2) atomicOr(&s[d + 2], w2);
}

// The same with one zero test for the whole field instead of one per dword: a
// lane whose field is 0 issues no atomic (sparse data packs many short fields
// into one dword, where atomics to the same address serialise), any other lane
// ORs every dword the field can touch, parts that are 0 included (q + 32 bits,
// q + 64 for a 64-bit field, must lie inside the array).  ubfe(x, 32 - sh, sh) is
// x >> (32 - sh), and 0 for sh == 0.
__device__ __forceinline__ void lds_or_bits(uint32_t *s, uint32_t q, uint32_t x) {
  if (x) {
    // the shift and the bit-field extract read only the low 5 bits of their
    // amounts, so q serves as the shift (q mod 32) and 32 - q as the extract offset
    // (width q mod 32 = 0 extracts nothing)
    uint32_t *p = s + (q >> 5);
    atomicOr(p, x << (q & 31u));
    atomicOr(p + 1, __builtin_amdgcn_ubfe(x, 32u - q, q));
  }
}

__device__ __forceinline__ void lds_or_bits(uint32_t *s, uint32_t q, uint16_t x) { lds_or_bits(s, q, (uint32_t)x); }

__device__ __forceinline__ void lds_or_bits(uint32_t *s, uint32_t q, uint64_t x) {
  const uint32_t d = q >> 5, sh = q & 31u;
  const uint32_t x0 = (uint32_t)x, x1 = (uint32_t)(x >> 32);
  if (x) {
    atomicOr(&s[d], x0 << sh);
    atomicOr(&s[d + 1], (x1 << sh) | __builtin_amdgcn_ubfe(x0, 32u - sh, sh));
    atomicOr(&s[d + 2], __builtin_amdgcn_ubfe(x1, 32u - sh, sh));
  }
}

// ------------------------------------------------------------------ global memory

// Output the kernel never reads back (decoded chunks, stream words, gathered rows):
// non-temporal stores (measured on the contiguous decoders: 0.73 -> 0.77 of the HBM
// peak for 64-bit chunks, 0.68 -> 0.75 for the GNN rows, 0.47 -> 0.64 for the
// sparse rows; the compressor, with non-temporal loads of its input, 3-4% faster).
template <typename V, typename X> __device__ __forceinline__ void store_nt(V *p, X v) {
  __builtin_nontemporal_store((V)v, p);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt16(void *p, const uint4 &v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, static_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store_nt8(void *p, const uint2 &v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, static_cast<u32x2 *>(p));
}

// Input read once (the compressor's chunks): a non-temporal load.
template <typename V> __device__ __forceinline__ V load_nt(const V *p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ uint4 load16(const uint8_t *src, uint64_t blk) {
  return *reinterpret_cast<const uint4 *>(src + blk * 16u);
}

// The 16-byte block that holds the last bytes of a buffer of nbytes bytes whose
// length is not a multiple of 16: read byte by byte, bytes past the end are 0.
__device__ __noinline__ uint4 load16_tail(const uint8_t *src, uint64_t nbytes, uint64_t blk) {
  const uint64_t b0 = blk * 16u;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (uint32_t j = 0; j < 16u; ++j)
    if (b0 + j < nbytes) w[j >> 2] |= (uint32_t)src[b0 + j] << (8u * (j & 3u));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint64_t atomic_load_agent(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_store_agent(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t atomic_or_agent(uint64_t *p, uint64_t v) {  // returns the former value
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_load_agent32(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void atomic_store_agent32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Decoupled look-back (Merrill & Garland, "Single-pass Parallel Prefix Scan with
// Decoupled Look-back", 2016).  Tile t publishes its aggregate agg (< 2^62) as soon
// as it knows it (lookback_publish), then finds its exclusive prefix by walking back
// over its predecessors' status words until one holds an inclusive prefix, adding
// the aggregates in between, and publishes its own inclusive prefix; the walk
// (lookback_finish) reads 64 predecessors per step, one per lane of a wavefront.
// Tile t is workgroup t: the dispatcher hands workgroups to the XCDs round-robin and
// starts each XCD's share in increasing order, so the lowest unfinished tile always
// has a slot (every earlier workgroup of its XCD has finished) and the wait chain
// makes progress.  (A single atomic ticket counter would also order them, but it
// serialises all workgroups on one address, at about 12 ns each.)
// Bounded (lookback_finish): a tile gives up after wait_limit polls of an
// unpublished predecessor, or at a poll that finds the abort flag control[1] set by
// another tile.  A tile that gives up sets control[1] and IBP_DEVERR_TIMEOUT, returns
// with timed_out set and publishes no prefix, so no successor takes a start bit from
// it: successors walk past its aggregate to the same unpublished predecessor, and
// either find it published later (their prefixes are then right) or give up too.
// lookback_publish: tile t's aggregate agg (tile 0: its inclusive prefix); one thread.
// Tile t's status word: word t >> lg of 16-word line t mod 2^lg (status_lg).
__device__ __forceinline__ uint64_t status_slot(uint64_t t, uint32_t lg) {
  return ((t & ((1ull << lg) - 1ull)) << 4) | (t >> lg);
}

__device__ inline void lookback_publish(uint64_t *status, uint32_t lg, uint64_t t, uint64_t agg) {
  atomic_store_agent(&status[status_slot(t, lg)], (t == 0 ? kFlagPrefix : kFlagAggregate) | agg);
}

// Summary of one window of 64 status words s (lane 0 the nearest predecessor):
//   kLbWait:   an unpublished predecessor lies before the window's first inclusive
//              prefix (the window must be read again later);
//   kLbPrefix: an inclusive prefix, with every nearer predecessor's aggregate
//              published: sum = that prefix plus those aggregates;
//   kLbAggs:   no prefix, every aggregate published: sum = their total.
enum : uint32_t { kLbWait = 0, kLbPrefix = 1, kLbAggs = 2 };
__device__ inline uint32_t lookback_window(uint64_t s, uint32_t lane, uint64_t &sum) {
  const uint64_t flag = s & ~kValueMask;
  const uint64_t pm = ballot(flag == kFlagPrefix);
  const uint64_t zm = ballot(flag == 0);
  const uint32_t first_p = pm ? (uint32_t)__builtin_ctzll(pm) : 64u;
  const uint64_t needed = first_p >= 63 ? ~0ull : ((2ull << first_p) - 1ull);
  sum = wave_sum64(lane <= first_p ? (s & kValueMask) : 0ull);
  return (zm & needed) ? kLbWait : (first_p < 64 ? kLbPrefix : kLbAggs);
}

// The rest of tile t's look-back, run by one wavefront: excl holds the sum of the
// windows before `base` (the nearest predecessor not yet accounted for); it walks
// back from base 64 at a time until an inclusive prefix, waiting (bounded) for
// unpublished predecessors, then publishes tile t's inclusive prefix and returns
// the exclusive one.
__device__ inline uint64_t lookback_finish(uint64_t *status, uint32_t lg, uint32_t *control, uint32_t *err, uint64_t t,
                                           int64_t base, uint64_t excl, uint64_t agg, uint32_t wait_limit,
                                           uint32_t lane, bool &timed_out) {
  timed_out = false;
  uint32_t spins = 0;
  while (base >= 0) {
    const int64_t j = base - (int64_t)lane;
    const uint64_t s = j >= 0 ? atomic_load_agent(&status[status_slot((uint64_t)j, lg)]) : kFlagPrefix;
    uint64_t sum;
    const uint32_t st = lookback_window(s, lane, sum);
    if (st == kLbWait) {
      // an unpublished predecessor: wait for it, within the bound
      ++spins;
      const bool over = spins > wait_limit;
      bool give_up = over;
      if (!over && (spins & 1023u) == 0u) give_up = atomic_load_agent32(&control[1]) != 0u;
      if (over && lane == 0) {
        atomic_store_agent32(&control[1], 1u);
        if (err) atomicOr(err, IBP_DEVERR_TIMEOUT);
      }
      if (ballot(give_up)) {
        timed_out = true;
        return 0;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    excl += sum;
    if (st == kLbPrefix) break;
    base -= 64;
  }
  if (lane == 0) atomic_store_agent(&status[status_slot(t, lg)], kFlagPrefix | ((excl + agg) & kValueMask));
  return excl;
}

}  // namespace dev

// Template run count for n runs: 1..8 unrolled, 0 = a loop over the runtime count.
// No free bits (Mask covers the chunk) takes the one-run form: the unused entry is
// zero (pmask 0, shift 0), so the deposit is 0 with no loop.
inline uint32_t runs_bucket(uint32_t n) { return n <= 8 ? (n == 0 ? 1u : n) : 0u; }

}  // namespace ibp
