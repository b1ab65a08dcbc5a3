// ibp_kernels.hip -- gfx950 kernels of the Invariant Bit Packing codec.
//
// Method: "Riduzione del Collo di Bottiglia della Memoria GPU con la Compressione
// Lossless per il ML" (gist.science, paper 2605.30728), section "Algoritmo Core",
// steps 1-3, and section "Integrazione del Sistema" (PCIe transfer mode).
// None of this is a dense contraction, so nothing here uses MFMA: the work is
// integer bit manipulation over streaming (HBM) or gathered (PCIe) data.  The
// tools are 64-lane ballots with mbcnt/popcount for prefix counts, LDS staging and
// bit assembly, and 16-byte global loads.
#include "ibp_internal.h"
#include "ibp.h"

namespace ibp {
namespace {

// ------------------------------------------------------------------ wave helpers

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below this one.
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc(uint64_t m) { return (uint32_t)__builtin_popcountll(m); }

__device__ __forceinline__ uint64_t low_lanes(uint32_t k) {  // bits [0, k), k <= 64
  return k >= 64 ? ~0ull : ((1ull << k) - 1ull);
}

// Orders this wavefront's LDS accesses around the call.  LDS instructions of one
// wavefront execute in program order, so only the compiler needs fencing.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

template <typename T> __device__ __forceinline__ T low_bits(uint32_t L) {
  constexpr uint32_t W = sizeof(T) * 8;
  return L >= W ? ~(T)0 : (T)(((T)1 << L) - (T)1);
}

// ------------------------------------------------------------------ bit moves

// Parallel bit extract of the free positions (payload of a matching chunk).
template <typename T> __device__ __forceinline__ T extract_free(T v, const CodecParams &p) {
  T out = 0;
  for (uint32_t r = 0; r < p.runs.n; ++r) out |= (v >> p.runs.shift[r]) & (T)p.runs.pmask[r];
  return out;
}

// Parallel bit deposit into the free positions (inverse of extract_free).
template <typename T> __device__ __forceinline__ T deposit_free(T x, const CodecParams &p) {
  T out = 0;
  for (uint32_t r = 0; r < p.runs.n; ++r) out |= (x & (T)p.runs.pmask[r]) << p.runs.shift[r];
  return out;
}

__device__ __forceinline__ uint32_t lds_bit(const uint32_t *s, uint32_t q) {
  return (s[q >> 5] >> (q & 31u)) & 1u;
}

// sizeof(T)*8 bits starting at local bit q (stream order, low bit first).
template <typename T> __device__ __forceinline__ T lds_field(const uint32_t *s, uint32_t q);

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

// OR an up-to-W-bit field (bits above its length already 0) into LDS at bit q.
__device__ __forceinline__ void lds_or_field(uint32_t *s, uint32_t q, uint32_t x) {
  const uint32_t d = q >> 5, sh = q & 31u;
  const uint32_t lo = x << sh;
  const uint32_t hi = sh ? (x >> (32u - sh)) : 0u;
  if (lo) atomicOr(&s[d], lo);
  if (hi) atomicOr(&s[d + 1], hi);
}

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

// 16-byte block blk of a buffer of nbytes bytes; bytes past the end read as 0.
__device__ __forceinline__ uint4 load_block(const uint8_t *src, uint64_t nbytes, uint64_t blk) {
  const uint64_t b0 = blk * 16u;
  if (b0 + 16u <= nbytes) return *reinterpret_cast<const uint4 *>(src + b0);
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

__device__ __forceinline__ uint32_t atomic_load_agent32(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ step 1: metadata

// Per-position one-counts of the sample chunks: every thread keeps W register
// counters, a workgroup sums them and writes one row of partial counts.
template <typename T>
__global__ void __launch_bounds__(kBlock) count_ones_kernel(MetaArgs a) {
  constexpr uint32_t W = sizeof(T) * 8;
  __shared__ uint32_t red[kWavesPerBlock][W];
  const T *in = static_cast<const T *>(a.in);
  uint32_t c[W];
#pragma unroll
  for (uint32_t b = 0; b < W; ++b) c[b] = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < a.n; i += stride) {
    const T v = in[i];
#pragma unroll
    for (uint32_t b = 0; b < W; ++b) c[b] += (uint32_t)((v >> b) & 1u);
  }
  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
  for (uint32_t b = 0; b < W; ++b) {
    const uint32_t s = wave_sum32(c[b]);
    if (lane == 0) red[wave][b] = s;
  }
  __syncthreads();
  if (threadIdx.x < W) {
    uint64_t s = 0;
    for (uint32_t w = 0; w < kWavesPerBlock; ++w) s += red[w][threadIdx.x];
    a.partial[(uint64_t)blockIdx.x * W + threadIdx.x] = s;
  }
}

// One wavefront: lane b sums the partial counts of position b and applies the
// threshold; the ballots of the per-lane verdicts are Mask and Bitval.
__global__ void __launch_bounds__(kWave) meta_finish_kernel(MetaArgs a) {
  const uint32_t b = threadIdx.x;
  uint64_t c1 = 0;
  if (b < a.W)
    for (uint32_t j = 0; j < a.blocks; ++j) c1 += a.partial[(uint64_t)j * a.W + b];
  const uint64_t c0 = a.n - c1;
  const uint64_t majority = c1 > c0 ? c1 : c0;
  const bool invariant = b < a.W && majority >= a.k;
  const uint64_t mask = ballot(invariant);
  const uint64_t bitval = ballot(invariant && c1 > c0);
  a.result[b] = b < a.W ? c1 : 0;
  if (b == 0) {
    a.result[64] = mask;
    a.result[65] = bitval;
  }
}

// ------------------------------------------------------------------ step 2: compression

// One workgroup per tile of G consecutive segments (about kEncTileChunks chunks).
//  1. take a tile ticket (tiles are numbered in start order, so every tile a
//     tile waits for is already running);
//  2. load the chunks, test the invariant bits, ballot the participation bits;
//  3. the tile's bit count follows from the number of matching chunks; publish
//     it, then wavefront 0 walks back over the predecessors' status words 64 at
//     a time (decoupled look-back) to get the tile's starting bit;
//  4. write the segment offsets, assemble the tile's bits in LDS with atomic ORs
//     (headers, then payloads = parallel bit extract or the raw chunk);
//  5. store the whole dwords; the dword shared with the previous tile is written
//     by this tile after OR-ing in the bits the previous tile handed over, and the
//     dword shared with the next tile is handed over instead of written.
template <typename T>
__global__ void __launch_bounds__(kBlock) encode_kernel(EncodeArgs a, CodecParams p) {
  constexpr uint32_t W = sizeof(T) * 8;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t *obuf = smem;
  uint64_t *bal = reinterpret_cast<uint64_t *>(smem + a.obuf_dw);  // 16 words
  uint32_t *pref = reinterpret_cast<uint32_t *>(bal + 16);          // 17 words
  __shared__ uint64_t s_excl;
  __shared__ uint32_t s_tile;
  __shared__ uint32_t s_failed;

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  if (tid == 0) s_tile = atomicAdd(&a.control[0], 1u);
  for (uint32_t d = tid; d < a.obuf_dw; d += kBlock) obuf[d] = 0u;
  __syncthreads();
  const uint64_t t = s_tile;
  if (t >= a.ntiles) return;  // more workgroups than tiles: cannot happen, grid == ntiles

  const uint64_t k0 = t * a.G;
  const uint64_t c0 = k0 * a.S;
  const uint32_t nsegt = (uint32_t)min((uint64_t)a.G, a.nseg - k0);
  const uint32_t nch = (uint32_t)min((uint64_t)a.tile_chunks, a.n_chunks - c0);
  const T *in = static_cast<const T *>(a.in) + c0;
  const T mask = (T)p.mask, bitval = (T)p.bitval;

  // 2. chunks and participation bits
  constexpr uint32_t kQ = kEncTileChunks / kBlock;  // passes of 256 chunks
  T v[kQ];
  uint32_t hbits = 0;
#pragma unroll
  for (uint32_t q = 0; q < kQ; ++q) {
    const uint32_t cl = q * kBlock + tid;
    v[q] = cl < nch ? in[cl] : (T)0;
  }
#pragma unroll
  for (uint32_t q = 0; q < kQ; ++q) {
    const uint32_t cl = q * kBlock + tid;
    const bool h = cl < nch && ((v[q] ^ bitval) & mask) == 0;
    hbits |= (uint32_t)h << q;
    const uint64_t B = ballot(h);
    if (lane == 0) bal[q * kWavesPerBlock + wave] = B;
  }
  __syncthreads();
  if (tid <= 16) {
    uint32_t s = 0;
    for (uint32_t j = 0; j < tid; ++j) s += popc(bal[j]);
    pref[tid] = s;
  }
  __syncthreads();
  // matching chunks among tile chunks [0, x)
  auto g = [&](uint32_t x) -> uint32_t {
    const uint32_t b = x >> 6, o = x & 63u;
    return pref[b] + (o ? popc(bal[b] & low_lanes(o)) : 0u);
  };
  const uint64_t agg = (uint64_t)nch * (W + 1) - (uint64_t)p.pc * pref[16];

  // 3. decoupled look-back
  if (wave == 0) {
    uint64_t excl = 0;
    bool timed_out = false;
    if (t == 0) {
      if (lane == 0) atomic_store_agent(&a.status[0], kFlagPrefix | agg);
    } else {
      if (lane == 0) atomic_store_agent(&a.status[t], kFlagAggregate | agg);
      int64_t base = (int64_t)t - 1;
      uint32_t spins = 0;
      while (true) {
        const int64_t j = base - (int64_t)lane;
        const uint64_t s = j >= 0 ? atomic_load_agent(&a.status[j]) : kFlagPrefix;
        const uint64_t flag = s & ~kValueMask;
        const uint64_t pm = ballot(flag == kFlagPrefix);
        const uint64_t zm = ballot(flag == 0);
        const uint32_t first_p = pm ? (uint32_t)__builtin_ctzll(pm) : 64u;
        const uint64_t needed = first_p >= 63 ? ~0ull : ((2ull << first_p) - 1ull);
        if ((zm & needed) && !timed_out) {
          // bounded wait: give up when another tile has aborted or after ~2^20 polls
          bool give_up = false;
          if ((++spins & 1023u) == 0u) give_up = atomic_load_agent32(&a.control[1]) != 0u;
          if (spins > (1u << 20)) {
            give_up = true;
            if (lane == 0) {
              __hip_atomic_store(&a.control[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if (a.err) atomicOr(a.err, IBP_DEVERR_TIMEOUT);
            }
          }
          timed_out = ballot(give_up) != 0;
          if (!timed_out) __builtin_amdgcn_s_sleep(1);
          continue;
        }
        excl += wave_sum64(lane <= first_p ? (s & kValueMask) : 0ull);
        if (first_p < 64) break;
        base -= 64;
      }
      if (lane == 0) atomic_store_agent(&a.status[t], kFlagPrefix | ((excl + agg) & kValueMask));
    }
    if (lane == 0) {
      s_excl = excl;
      s_failed = timed_out ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint64_t excl = s_excl;
  // a tile that gave up waiting has no valid start bit: it must not store anything
  // that depends on it (its neighbours see the abort flag and give up as well)
  const bool failed = s_failed != 0u;

  // 4a. segment offsets
  if (failed) {
    if (tid == 0) atomic_store_agent(&a.tails[t], kTailReady);
    return;
  }
  for (uint32_t r = tid; r < nsegt; r += kBlock)
    a.off[k0 + r] = excl + (uint64_t)r * a.S * (W + 1) - (uint64_t)p.pc * g(r * a.S);
  if (t == a.ntiles - 1 && tid == 0) a.off[a.nseg] = excl + agg;

  // 4b. pack into LDS; bit 0 of obuf is stream bit (excl & ~31)
  const uint32_t lb0 = (uint32_t)(excl & 31u);
#pragma unroll
  for (uint32_t q = 0; q < kQ; ++q) {
    const uint32_t cl = q * kBlock + tid;
    if (cl < nch) {
      uint32_t r, i;
      if (a.s_log2 != kNotPow2) {
        r = cl >> a.s_log2;
        i = cl & (a.S - 1u);
      } else {
        r = cl / a.S;
        i = cl - r * a.S;
      }
      const uint32_t s0 = r * a.S;
      const uint32_t m = min(a.S, nch - s0);
      const uint32_t gs = g(s0);
      const uint32_t segbase = lb0 + s0 * (W + 1) - p.pc * gs;
      const bool h = (hbits >> q) & 1u;
      if (h) atomicOr(&obuf[(segbase + i) >> 5], 1u << ((segbase + i) & 31u));
      const uint32_t pos = segbase + m + i * W - p.pc * (g(cl) - gs);
      const T payload = h ? extract_free(v[q], p) : v[q];
      lds_or_field(obuf, pos, payload);
    }
  }
  __syncthreads();

  // 5. store; hand over the shared last dword, complete the shared first dword
  const uint32_t nd = (uint32_t)((lb0 + agg + 31u) >> 5);
  const bool has_head = lb0 != 0u;
  const bool has_tail = ((lb0 + agg) & 31u) != 0u;
  const bool last = t == a.ntiles - 1;
  uint32_t *gdst = a.stream + (excl >> 5);
  for (uint32_t d = tid; d < nd; d += kBlock) {
    const bool skip = (d == 0 && has_head) || (d == nd - 1 && has_tail && !last);
    if (!skip) gdst[d] = obuf[d];
  }
  if (tid == 0) {
    if (has_tail && !last) atomic_store_agent(&a.tails[t], kTailReady | obuf[nd - 1]);
    if (has_head) {
      uint64_t prev = 0;
      uint32_t spins = 0;
      while (true) {
        prev = atomic_load_agent(&a.tails[t - 1]);
        if (prev & kTailReady) break;
        if ((++spins & 1023u) == 0u && atomic_load_agent32(&a.control[1]) != 0u) break;
        if (spins > (1u << 20)) {
          __hip_atomic_store(&a.control[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (a.err) atomicOr(a.err, IBP_DEVERR_TIMEOUT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      gdst[0] = obuf[0] | (uint32_t)prev;
    }
  }
}

__global__ void __launch_bounds__(kBlock) zero_kernel(uint64_t *p, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// ------------------------------------------------------------------ step 3: decompression

// Each wavefront decodes one tile of G units (segments for the contiguous
// decode, rows for the gather):
//  a. read the units' bit ranges from the offset table and check them;
//  b. stage the compressed bits in LDS with 16-byte loads, all issued before any
//     LDS write (the contiguous tile is one range; a gather stages each row in
//     its own slot);
//  c. per pass of 64 chunks: each lane reads its participation bit, a ballot +
//     mbcnt gives the number of compressed chunks before it in its segment, hence
//     its payload offset (every chunk before it costs W bits, minus popcount(Mask)
//     for each compressed one); read the payload from LDS, deposit it into the
//     free positions and OR in Bitval, or take it raw; store.
template <typename T, bool kGather>
__global__ void __launch_bounds__(kBlock) decode_kernel(DecodeArgs a, CodecParams p) {
  constexpr uint32_t W = sizeof(T) * 8;
  constexpr uint32_t kBad = 0xFFFFFFFFu;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
  const uint64_t u0 = ((uint64_t)blockIdx.x * kWavesPerBlock + wave) * a.G;
  if (u0 >= a.n_units) return;
  const uint32_t nu = (uint32_t)min((uint64_t)a.G, a.n_units - u0);
  uint32_t *stg = smem + (uint64_t)wave * a.wave_dw;
  uint32_t *lbeg = stg + a.stage_dw;
  uint32_t *lend = lbeg + a.G;
  uint32_t *gseg = lend + a.G;
  const uint64_t chunk0 = u0 * a.S;
  const uint32_t nch = (uint32_t)min((uint64_t)nu * a.S, a.n_chunks - chunk0);
  uint32_t errbits = 0;

  if constexpr (!kGather) {
    // a. the tile's range [A, B) and its segments
    const uint64_t A = a.off[u0], B = a.off[u0 + nu];
    const bool tile_ok = A <= B && B - A <= (uint64_t)nch * (W + 1) && B <= a.stream_bytes * 8u;
    if (!tile_ok) {
      if (lane == 0 && a.err) atomicOr(a.err, IBP_DEVERR_CORRUPT);
      return;
    }
    const uint64_t base = A & ~127ull;
    for (uint32_t r = lane; r < nu; r += kWave) {
      const uint64_t x = a.off[u0 + r], y = a.off[u0 + r + 1];
      const uint64_t m = min((uint64_t)a.S, a.n_chunks - (u0 + r) * a.S);
      const bool good = A <= x && x <= y && y <= B && y - x >= m && y - x <= m * (W + 1);
      lbeg[r] = good ? (uint32_t)(x - base) : kBad;
      lend[r] = good ? (uint32_t)(y - base) : kBad;
      if (!good) errbits |= IBP_DEVERR_CORRUPT;
    }
    // b. stage
    const uint64_t blk0 = A >> 7;
    const uint32_t nb = (uint32_t)(((B + 127u) >> 7) - blk0);
    for (uint32_t j0 = 0; j0 < nb; j0 += 4 * kWave) {
      uint4 tmp[4];
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) {
        const uint32_t j = j0 + u * kWave + lane;
        if (j < nb) tmp[u] = load_block(a.stream, a.stream_bytes, blk0 + j);
      }
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) {
        const uint32_t j = j0 + u * kWave + lane;
        if (j < nb) *reinterpret_cast<uint4 *>(stg + 4 * j) = tmp[u];
      }
    }
  } else {
    uint64_t *ufirst = reinterpret_cast<uint64_t *>(gseg + a.G + (a.G & 1u));
    uint32_t *unb = reinterpret_cast<uint32_t *>(ufirst + a.G);
    // a. rows
    for (uint32_t r = lane; r < nu; r += kWave) {
      const int64_t id = a.ids[u0 + r];
      bool good = id >= 0 && (uint64_t)id < a.nseg;
      if (!good) errbits |= IBP_DEVERR_BAD_ID;
      uint64_t x = 0, y = 0;
      if (good) {
        x = a.off[id];
        y = a.off[id + 1];
        const bool sane = x <= y && y <= a.stream_bytes * 8u && y - x >= a.S &&
                          y - x <= (uint64_t)a.S * (W + 1);
        if (!sane) {
          good = false;
          errbits |= IBP_DEVERR_CORRUPT;
        }
      }
      const uint32_t slot = r * a.slot_dw * 32u;
      lbeg[r] = good ? slot + (uint32_t)(x & 127u) : kBad;
      lend[r] = good ? slot + (uint32_t)(y - (x & ~127ull)) : kBad;
      ufirst[r] = x >> 7;
      unb[r] = good ? (uint32_t)(((y + 127u) >> 7) - (x >> 7)) : 0u;
    }
    wave_lds_sync();
    // b. stage every row into its slot
    const uint32_t sb = a.slot_dw / 4u;
    const uint32_t total = nu * sb;
    for (uint32_t f0 = 0; f0 < total; f0 += 4 * kWave) {
      uint4 tmp[4];
      uint32_t dst[4];
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) {
        const uint32_t f = f0 + u * kWave + lane;
        const uint32_t r = f / sb, j = f - r * sb;
        dst[u] = kBad;
        if (f < total && j < unb[r]) {
          tmp[u] = load_block(a.stream, a.stream_bytes, ufirst[r] + j);
          dst[u] = r * a.slot_dw + 4u * j;
        }
      }
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u)
        if (dst[u] != kBad) *reinterpret_cast<uint4 *>(stg + dst[u]) = tmp[u];
    }
  }
  wave_lds_sync();

  // c. decode
  const T cmask = low_bits<T>(W - p.pc);
  const T bitval = (T)p.bitval;
  T *out = static_cast<T *>(a.out) + chunk0;
  uint32_t running = 0;  // compressed chunks among tile chunks [0, p0)
  for (uint32_t p0 = 0; p0 < nch; p0 += kWave) {
    const uint32_t cl = p0 + lane;
    const bool valid = cl < nch;
    uint32_t r, i;
    if (a.s_log2 != kNotPow2) {
      r = cl >> a.s_log2;
      i = cl & (a.S - 1u);
    } else {
      r = cl / a.S;
      i = cl - r * a.S;
    }
    const uint32_t lb = valid ? lbeg[r] : kBad;
    const bool ok = lb != kBad;
    uint32_t m = a.S;
    if constexpr (!kGather) m = (uint32_t)min((uint64_t)a.S, a.n_chunks - (chunk0 + (uint64_t)r * a.S));
    const uint32_t h = ok ? lds_bit(stg, lb + i) : 0u;
    const uint64_t H = ballot(h != 0u);
    const uint32_t g_cl = running + count_below(H);
    const uint32_t s0 = r * a.S;
    uint32_t g_start;
    if (s0 >= p0) {
      g_start = running + popc(H & low_lanes(s0 - p0));
    } else {
      g_start = valid ? gseg[r] : 0u;
    }
    if (valid && i == 0) gseg[r] = g_cl;
    const uint32_t pos = ok ? lb + m + i * W - p.pc * (g_cl - g_start) : 0u;
    T x = lds_field<T>(stg, pos);
    x &= h ? cmask : ~(T)0;
    const T val = h ? (deposit_free(x, p) | bitval) : x;
    if (ok) {
      out[cl] = val;
      if (i == m - 1 && pos + (h ? W - p.pc : W) != lend[r]) errbits |= IBP_DEVERR_CORRUPT;
    }
    running += popc(H);
    wave_lds_sync();
  }
  if (errbits && a.err) atomicOr(a.err, errbits);
}

// Uncompressed gather baseline: row j = row ids[j], 16 bytes per lane.
__global__ void __launch_bounds__(kBlock) raw_gather_kernel(RawGatherArgs a) {
  const uint64_t total = a.n_ids * a.row_blocks;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t f = (uint64_t)blockIdx.x * kBlock + threadIdx.x; f < total; f += stride) {
    const uint64_t j = f / a.row_blocks, b = f - j * a.row_blocks;
    const int64_t id = a.ids[j];
    if (id < 0 || (uint64_t)id >= a.n_rows) {
      if (b == 0 && a.err) atomicOr(a.err, IBP_DEVERR_BAD_ID);
      continue;
    }
    const uint4 x = reinterpret_cast<const uint4 *>(a.src)[(uint64_t)id * a.row_blocks + b];
    reinterpret_cast<uint4 *>(a.out)[f] = x;
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

static inline uint64_t host_min(uint64_t x, uint64_t y) { return x < y ? x : y; }

hipError_t launch_meta(const MetaArgs &a, hipStream_t s) {
  if (a.n) {
    if (a.W == 32)
      hipLaunchKernelGGL(count_ones_kernel<uint32_t>, dim3(a.blocks), dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL(count_ones_kernel<uint64_t>, dim3(a.blocks), dim3(kBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(meta_finish_kernel, dim3(1), dim3(kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, const CodecParams &p, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  // clear the ticket, abort flag, status and hand-over words (a kernel, not a
  // memset node, so the sequence stays valid inside a captured graph)
  const uint64_t nzero = 2 * a.ntiles + 1;  // control (8 bytes) + status + tails, contiguous
  const uint32_t zb = (uint32_t)host_min((nzero + kBlock - 1) / kBlock, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(zb), dim3(kBlock), 0, s, reinterpret_cast<uint64_t *>(a.control), nzero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t shmem = (size_t)a.obuf_dw * 4 + 16 * 8 + 17 * 4;
  if (a.ntiles > 0x7FFFFFFFull) return hipErrorInvalidValue;
  if (p.W == 32)
    hipLaunchKernelGGL(encode_kernel<uint32_t>, dim3((uint32_t)a.ntiles), dim3(kBlock), shmem, s, a, p);
  else
    hipLaunchKernelGGL(encode_kernel<uint64_t>, dim3((uint32_t)a.ntiles), dim3(kBlock), shmem, s, a, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, const CodecParams &p, bool gather, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  const uint64_t tiles = (a.n_units + a.G - 1) / a.G;
  const uint64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const size_t shmem = (size_t)a.wave_dw * 4 * kWavesPerBlock;
  const dim3 grid((uint32_t)blocks), block(kBlock);
  if (p.W == 32) {
    if (gather)
      hipLaunchKernelGGL((decode_kernel<uint32_t, true>), grid, block, shmem, s, a, p);
    else
      hipLaunchKernelGGL((decode_kernel<uint32_t, false>), grid, block, shmem, s, a, p);
  } else {
    if (gather)
      hipLaunchKernelGGL((decode_kernel<uint64_t, true>), grid, block, shmem, s, a, p);
    else
      hipLaunchKernelGGL((decode_kernel<uint64_t, false>), grid, block, shmem, s, a, p);
  }
  return hipGetLastError();
}

hipError_t launch_zero(uint64_t *p, uint64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint32_t blocks = (uint32_t)host_min((n + kBlock - 1) / kBlock, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(kBlock), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_raw_gather(const RawGatherArgs &a, hipStream_t s) {
  const uint64_t total = a.n_ids * a.row_blocks;
  if (total == 0) return hipSuccess;
  const uint32_t blocks = (uint32_t)host_min((total + kBlock - 1) / kBlock, 65536);
  hipLaunchKernelGGL(raw_gather_kernel, dim3(blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace ibp
