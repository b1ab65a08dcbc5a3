// ibp_encode.hip -- step 2 of the IBP codec on gfx950: compression in one pass
// ("Riduzione del Collo di Bottiglia della Memoria GPU con la Compressione
// Lossless per il ML", section "Algoritmo Core", Compressione).
//
// A chunk whose Mask bits equal Bitval loses them (the remaining bits close up
// towards bit 0); every chunk gets a participation bit.  The participation bits
// of a segment are written first, as its header, then the payloads.  Each
// workgroup sizes its tile, obtains the tile's starting bit through a decoupled
// look-back over its predecessors (Merrill & Garland, "Single-pass Parallel
// Prefix Scan with Decoupled Look-back", 2016), and packs the tile in LDS.
#include <type_traits>
#include <utility>

#include "ibp_device.h"

namespace ibp {
namespace {

using namespace dev;

enum : uint32_t {
  kModeGeneral = 0,  // any S
  kModeSmallS = 1,   // 64 % S == 0: each 64-chunk block holds 64/S whole segments
  kModeLargeS = 2,   // S % 64 == 0: each 64-chunk block lies inside one segment
};

// One workgroup per tile of G consecutive segments (about 16 chunks per thread,
// 32 in the W = 16 pair form).
//  1. tile t = workgroup index (see the look-back in ibp_device.h for why the order holds);
//  2. load the chunks (16 per thread, 64 consecutive per wavefront per pass),
//     test the invariant bits and ballot the participation bits; clear the LDS
//     image while the loads are in flight;
//  3. a wave-wide scan of the ballot popcounts gives the number of compressed
//     chunks before every 64-chunk block, hence every segment's size and the
//     tile's, which is published at once for the successors' look-back;
//  4. assemble the tile's bits with atomic ORs in an LDS image that starts at the
//     tile's own first bit (payloads = parallel bit extract or the raw chunk;
//     the headers of S >= 64 segments as whole 64-bit ballots, once per tile);
//  5. wavefront 0 walks back over the predecessors' status words 64 at a time
//     (decoupled look-back) to get the tile's first bit;
//  6. write the segment offsets;
//  7. store the image shifted to the first bit's place in its 16-byte block
//     (interior 16-byte stores from two aligned LDS reads); a dword shared with
//     a neighbouring tile is written by whichever of the two tiles comes second:
//     each ORs its bits of the dword and its flag into the boundary's hand-over
//     word, and the one whose OR returns the other's flag writes the dword.
//     No tile waits for a neighbour's store.
// The per-chunk prefix count has the decoder's three forms (S a multiple of 64,
// S dividing 64, any S).
//
// kPair (W = 16, one Mask, S a multiple of 64, input 4-byte aligned): a lane
// takes two consecutive chunks as one 32-bit word per pass (128 chunks per
// wavefront), tests both, and ballots the even and the odd chunks.  A 64-chunk
// block's word holds its 32 even chunks' bits low and its 32 odd chunks' bits
// high (its popcount, all the prefix counts need, is the same) and is interleaved
// into stream order only where the header is written.  The free
// bits of both chunks are extracted together on the pair word (each run's mask
// in both halves: a run never crosses a half), and the two payloads go into LDS
// as one field of at most 32 bits, half the LDS atomics of one chunk per lane.
//
// kPos: position-dependent metadata.  Chunk position i of a segment has its own
// Mask_i / Bitval_i (tables in device memory, copied to LDS), so a matching chunk
// saves popcount(Mask_i) bits instead of a constant: the count of compressed
// chunks times popcount(Mask) becomes a prefix sum of per-chunk savings (a wave
// scan per 64-chunk block plus a scan over the blocks), and the extraction walks
// the runs of each lane's own free positions.
// Bits 0..31 of e at the even positions of the result, of o at the odd ones.
__device__ __forceinline__ uint64_t interleave32(uint32_t e, uint32_t o) {
  auto spread = [](uint64_t x) {
    x = (x | (x << 16)) & 0x0000FFFF0000FFFFull;
    x = (x | (x << 8)) & 0x00FF00FF00FF00FFull;
    x = (x | (x << 4)) & 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x << 2)) & 0x3333333333333333ull;
    return (x | (x << 1)) & 0x5555555555555555ull;
  };
  return spread(e) | (spread(o) << 1);
}

// The pair form asks for 8 wavefronts per SIMD (its 16 unrolled passes otherwise
// take enough scalar registers to allow only 7: 1.28 -> 1.11 ms per 2^30 chunks).
template <typename T, uint32_t kMode, uint32_t NR, bool kPos, bool kPair = false, uint32_t kHalves = 1, bool kBig = false>
__global__ void __launch_bounds__(enc_threads(kPos, sizeof(T) * 8, kBig), (kPair || (kHalves == 2 && !kPos)) ? 8 : 1)
    encode_kernel(EncodeArgs a, CodecParams p) {
  static_assert(!kPair || (sizeof(T) == 2 && kMode == 2 && !kPos), "pairs: W = 16, S a multiple of 64, one Mask");
  static_assert(enc_threads(kPos, sizeof(T) * 8) > kWave, "the two hand-over atomics come from two wavefronts");
  static_assert(kHalves == 1 || (!kPair && kMode != kModeGeneral), "halves: S a power of two");
  static_assert(!kBig || (kHalves == 2 && sizeof(T) == 8), "1024-thread tiles: 64-bit chunks in halves");
  constexpr uint32_t W = sizeof(T) * 8;
  constexpr uint32_t kThreads = enc_threads(kPos, W, kBig);
  constexpr uint32_t kWaves = kThreads / kWave;
  constexpr uint32_t kTile = enc_tile_chunks(kPos, kPair, W, kHalves, kBig);
  constexpr uint32_t kQ = kTile / kThreads;  // passes of kThreads chunks
  constexpr uint32_t kBal = kTile / kWave;   // 64-chunk blocks per tile
  constexpr uint32_t kPer = (kBal + kWave - 1) / kWave;  // 64-chunk blocks per lane of the prefix scan
  static_assert(kBal <= kWave || kBal == kPer * kWave, "whole blocks per lane of the prefix scan");
  constexpr uint32_t kQP = kPair ? kQ / 2 : 1;  // kPair: passes of kThreads chunk pairs
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t *obuf = smem;
  uint64_t *bal = reinterpret_cast<uint64_t *>(smem + a.obuf_dw);  // kBal words
  uint32_t *pref = reinterpret_cast<uint32_t *>(bal + kBal);        // kBal + 1 words
  // kPos: Mask_i / Bitval_i tables (S words each) and each chunk's inclusive prefix
  // of saved bits within its 64-chunk block
  uint64_t *mtab = reinterpret_cast<uint64_t *>(pref + kBal + 2);
  uint64_t *btab = mtab + (kPos ? a.S : 0u);
  uint16_t *wpre = reinterpret_cast<uint16_t *>(btab + (kPos ? a.S : 0u));
  __shared__ uint64_t s_excl;
  __shared__ uint32_t s_failed;
  __shared__ uint32_t s_carry;  // kHalves: the first half's bits of the dword both halves share

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = uniform(tid / kWave);
  const uint64_t t = blockIdx.x;  // grid == ntiles

  const uint64_t k0 = t * a.G;
  const uint64_t c0 = k0 * a.S;
  const uint32_t nsegt = (uint32_t)min((uint64_t)a.G, a.nseg - k0);
  const uint32_t nch = (uint32_t)min((uint64_t)a.tile_chunks, a.n_chunks - c0);
  const T *in = static_cast<const T *>(a.in) + c0;
  const T mask = (T)p.mask, bitval = (T)p.bitval;
  const uint32_t pc = p.pc;

  // 2. chunks, participation bits; clear the image meanwhile
  T v[kQ];
  uint32_t v2[kQP];  // kPair: chunks 2 (q kThreads + tid) and the next one
  if constexpr (kPair) {
    const uint32_t *in2 = reinterpret_cast<const uint32_t *>(in);
    if (nch == kTile) {
#pragma unroll
      for (uint32_t q = 0; q < kQP; ++q) v2[q] = load_nt(&in2[q * kThreads + tid]);
    } else {
#pragma unroll
      for (uint32_t q = 0; q < kQP; ++q) {
        const uint32_t c = 2u * (q * kThreads + tid);
        v2[q] = c + 1u < nch ? in2[c / 2u] : (c < nch ? (uint32_t)in[c] : 0u);
      }
    }
  } else if (nch == kTile) {  // every tile but possibly the last: no bounds tests
#pragma unroll
    for (uint32_t q = 0; q < kQ; ++q) v[q] = load_nt(&in[q * kThreads + tid]);
  } else {
#pragma unroll
    for (uint32_t q = 0; q < kQ; ++q) {
      const uint32_t cl = q * kThreads + tid;
      v[q] = cl < nch ? in[cl] : (T)0;
    }
  }
  for (uint32_t d = 4 * tid; d < a.obuf_dw; d += 4 * kThreads)
    *reinterpret_cast<uint4 *>(obuf + d) = make_uint4(0u, 0u, 0u, 0u);
  uint32_t ip[kQ];   // kPos: position of chunk q * kThreads + tid in its segment (tiles start on a segment)
  uint32_t svx[kQ];  // kPos: saved bits of the earlier chunks of its 64-chunk block
  // kPos: whether some position's free bits are not one run from bit 0 (per 32-bit
  // half at W = 64).  When none is, a matching chunk's payload is its value AND its
  // free bits; the packing passes are instantiated for both cases, chosen once.
  bool multi = false;
  if constexpr (kPos) {
    const uint64_t full = W >= 64 ? ~0ull : ((1ull << W) - 1ull);
    int mine = 0;
    for (uint32_t i = tid; i < a.S; i += kThreads) {
      const uint64_t m = a.pmask[i] & full;
      mtab[i] = m;
      btab[i] = a.pbitval[i] & m;
      const uint64_t F = ~m & full;
      const uint32_t Flo = (uint32_t)F, Fhi = (uint32_t)(F >> 32);
      if ((Flo & (Flo + 1u)) != 0u || (Fhi & (Fhi + 1u)) != 0u) mine = 1;
    }
    const uint32_t step = kThreads % a.S;
    uint32_t i0 = tid % a.S;
#pragma unroll
    for (uint32_t q = 0; q < kQ; ++q) {
      ip[q] = i0;
      i0 += step;
      if (i0 >= a.S) i0 -= a.S;
    }
    multi = uniform((uint32_t)__syncthreads_or(mine)) != 0u;
  }
  uint64_t B[kQ];  // this wavefront's participation ballots, one per pass
  // One Mask with more than 16 passes (32-bit chunks in 16,384-chunk tiles): pass
  // q's participation ballot is taken again where it is needed rather than held in
  // scalar registers (32 ballots do not fit beside the rest and are spilled to
  // vector-register lanes, four instructions per pass).  The lanes past the
  // tile's end (a scalar mask; none in a full tile) take no part.
  constexpr bool kRetake = !kPos && !kPair && kQ > 16;
  const bool full_tile = nch == kTile;
  auto match_ballot = [&](uint32_t q) -> uint64_t {
    const uint64_t b = ballot(((v[q] ^ bitval) & mask) == 0);
    if (full_tile) return b;
    const uint32_t base = q * kThreads + wave * kWave;
    return b & (base >= nch ? 0ull : low_lanes(min(nch - base, kWave)));
  };
  // kPair: participation ballots of the even (E) and the odd (O) chunks of pass q's
  // pairs, from one XOR-AND of the pair word with Bitval and Mask in both halves; lanes
  // whose chunk lies past the tile's end take no part (scalar masks; none in a full
  // tile).  Taken again when packing rather than held across the barriers.
  // Mask and Bitval in both halves are held in vector registers (opaque to the
  // compiler): with both in scalar registers, the one three-operand logic op per
  // pass would need two of them, more than one instruction may read.
  // The low-half test compares against a zero held the same way (the compare that
  // selects a half takes no constant operand).
  uint32_t m2 = (uint32_t)mask * 0x10001u, b2 = (uint32_t)bitval * 0x10001u, zero = 0u;
  if constexpr (kPair) asm volatile("" : "+v"(m2), "+v"(b2), "+v"(zero));
  auto pair_ballots = [&](uint32_t q, uint64_t &E, uint64_t &O) {
    uint32_t d = (v2[q] ^ b2) & m2;
    asm("" : "+v"(d));  // one three-operand logic op, both tests on its result
    E = ballot((d & 0xFFFFu) == zero);
    O = ballot(d < 0x10000u);
    if (!full_tile) {
      const uint32_t cb = 2u * (q * kThreads + wave * kWave);  // the pass's first chunk
      const uint32_t left = uniform(cb < nch ? nch - cb : 0u);  // chunks of the pass in the tile
      E &= low_lanes(min((left + 1u) >> 1, kWave));
      O &= low_lanes(min(left >> 1, kWave));
    }
  };
  if constexpr (kPair) {
    // the span's two 64-chunk blocks are lanes 0-31 and 32-63: words 2p and 2p + 1
    // hold the even and the odd ballot whole, low halves for the first block (the
    // wavefront's base address in a vector register, the pass in the offset field)
    uint32_t bw = 2u * wave;
    asm volatile("" : "+v"(bw));
#pragma unroll
    for (uint32_t q = 0; q < kQP; ++q) {
      uint64_t E, O;
      pair_ballots(q, E, O);
      if (lane == 0) {
        bal[bw + 2u * q * kWaves] = E;
        bal[bw + 2u * q * kWaves + 1u] = O;
      }
    }
  }
#pragma unroll
  for (uint32_t q = 0; q < (kPair ? 0u : kQ); ++q) {
    const uint32_t cl = q * kThreads + tid;
    if constexpr (kPos) {
      const uint64_t m = mtab[ip[q]];
      const bool h = cl < nch && ((v[q] ^ (T)btab[ip[q]]) & (T)m) == 0;
      B[q] = ballot(h);
      // saved bits: an inclusive wave scan over the block's 64 chunks
      const uint32_t sv = h ? popc(m) : 0u;
      const uint32_t x = wave_incl_scan(sv);
      svx[q] = x - sv;
      // segments of a multiple of 64 chunks start on a block, so the per-chunk
      // prefix is neither needed nor allocated there
      if constexpr (kMode != kModeLargeS) wpre[cl] = (uint16_t)x;
      if (lane == kWave - 1) bal[q * kWaves + wave] = x;  // the block's saved bits
    } else {
      const uint64_t b = match_ballot(q);
      if constexpr (!kRetake) B[q] = b;
      if (lane == 0) bal[q * kWaves + wave] = b;
    }
  }
  // Every input load has been consumed.  An explicit wait for all vector memory
  // operations here (none is outstanding) lets the compiler know it: otherwise,
  // where the full-tile and tail-tile load paths join, it places a vmcnt(0) wait in
  // the packing loop, which would also wait for the publish store and the early
  // look-back read issued after this point.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  // 3. compressed chunks before each 64-chunk block
  if (wave == 0) {
    // lane l sums blocks [kPer l, kPer l + kPer)
    uint32_t cs[kPer], c = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
      const uint32_t b = kPer * lane + k;
      if constexpr (kPair) {
        const uint32_t sh = (b & 1u) * 32u;
        cs[k] = b < kBal ? popc((uint32_t)(bal[b & ~1u] >> sh)) + popc((uint32_t)(bal[b | 1u] >> sh)) : 0u;
      } else {
        cs[k] = b < kBal ? (kPos ? (uint32_t)bal[b] : popc(bal[b])) : 0u;
      }
      c += cs[k];
    }
    uint32_t x = wave_incl_scan(c) - c;
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
      const uint32_t b = kPer * lane + k;
      if (b < kBal) pref[b] = x;
      x += cs[k];
    }
    if (lane == kWave - 1) pref[kBal] = x;
  }
  __syncthreads();
  // compressed chunks among tile chunks [0, x), any x <= tile size (kPair: x a
  // multiple of 64, segments of a multiple of 64 chunks)
  auto g = [&](uint32_t x) -> uint32_t {
    const uint32_t b = x >> 6, o = kPair ? 0u : x & 63u;
    return pref[b] + (o ? popc(bal[b] & low_lanes(o)) : 0u);
  };
  // bits saved by the matching chunks among tile chunks [0, x), any x < tile size
  // (position metadata with S a multiple of 64: segment starts only)
  auto cost = [&](uint32_t x) -> uint32_t {
    if constexpr (kPos) {
      const uint32_t b = x >> 6, o = x & 63u;
      if constexpr (kMode == kModeLargeS) return pref[b];  // x is a segment start: o == 0
      return pref[b] + (o ? (uint32_t)wpre[x - 1] : 0u);
    } else {
      return pc * g(x);
    }
  };
  const uint64_t agg = (uint64_t)nch * (W + 1) - (kPos ? (uint64_t)pref[kBal] : (uint64_t)pc * pref[kBal]);

  // publish the tile's size at once, so successors can look back past it while
  // this tile packs
  if (tid == 0) lookback_publish(a.status, a.st_lg, t, agg);

  // 4. pack into LDS, from bit 0 of the image (the tile's first bit); the store
  //    shifts the image to the tile's place in the stream.  Segment s0's header
  //    starts at image bit s0 (W + 1) - (bits saved before s0); its payloads
  //    follow the m header bits, so chunk cl's payload starts at
  //    s0 + m + cl W - (bits saved by the tile chunks before cl).
  const uint32_t lane_bits = lane * W;
  // lane l holds the values of 64-chunk blocks l, 64 + l, ...
  uint32_t my_pref[kPer];
#pragma unroll
  for (uint32_t k = 0; k < kPer; ++k) my_pref[k] = kWave * k + lane <= kBal ? pref[kWave * k + lane] : 0u;
  // the prefix of block b0 + m wave, where b0 = m q kWaves is a constant once the
  // passes are unrolled: m kWaves divides 64 and wave < kWaves, so every
  // wavefront's block lies in my_pref[b0 / 64], lane (b0 mod 64) + m wave, and the
  // lookup is one v_readlane
  static_assert(kWave % (2 * kWaves) == 0, "two blocks per wavefront fit one lane row");
  auto pref_at = [&](uint32_t b0, uint32_t m) -> uint32_t {
    const uint32_t l = (b0 & 63u) + m * wave;
    uint32_t v = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k)
      if ((b0 >> 6) == k) v = (uint32_t)__builtin_amdgcn_readlane((int)my_pref[k], (int)l);
    return v;
  };
  auto seg_start = [&](uint32_t c) -> uint32_t {  // first chunk of the segment holding tile chunk c
    return a.s_log2 != kNotPow2 ? (c >> a.s_log2) << a.s_log2 : (c / a.S) * a.S;
  };
  const uint32_t i_lane = lane & (a.S - 1u);                   // small-S: index in segment
  const uint64_t seg_below = low_lanes(lane & ~(a.S - 1u));     // small-S: earlier segments' lanes
  // kPair: per-lane terms of the passes kept in vector registers (opaque, so they
  // are not formed again from scalar values in every pass): the lane's first
  // chunk's bit if every chunk before it were raw (2 W per lane), -popcount(Mask)
  // for the one multiply-add, and W - popcount(Mask), a compressed chunk's payload
  uint32_t lane2w = lane * 2u * W, wpc = W - pc;
  int32_t npc = -(int32_t)pc;
  if constexpr (kPair) asm volatile("" : "+v"(lane2w), "+v"(wpc), "+v"(npc));
  // kPair: the passes, in one copy for S a multiple of 128 (a pass's two 64-chunk
  // blocks lie in one segment, whose start and length are then scalar) and one for
  // S = 64 mod 128 (the blocks may lie in different segments)
  auto pair_passes = [&](auto one_seg) __attribute__((always_inline)) {
#pragma unroll
    for (uint32_t q = 0; q < kQP; ++q) {
      const uint32_t blk = 2u * (q * kWaves + wave);  // first of the span's two 64-chunk blocks
      const uint32_t cb = blk * kWave;
      if (cb >= nch) continue;  // uniform
      const uint32_t s_lo = seg_start(cb);
      uint32_t s0 = s_lo;
      if constexpr (!decltype(one_seg)::value) {
        const uint32_t s_hi = seg_start(min(cb + kWave, nch - 1u));
        s0 = lane < 32u ? s_lo : s_hi;
      }
      const uint32_t m = min(a.S, nch - s0);
      uint64_t E, O;
      pair_ballots(q, E, O);
      const bool h0 = __builtin_amdgcn_inverse_ballot_w64(E), h1 = __builtin_amdgcn_inverse_ballot_w64(O);
      // compressed chunks before the lane's pair: the block prefix (in the scalar
      // part), then the even and the odd chunks of the lower lanes, accumulated by
      // the lane-count instructions
      uint32_t cnt = __builtin_amdgcn_mbcnt_lo((uint32_t)E, 0u);
      cnt = __builtin_amdgcn_mbcnt_hi((uint32_t)(E >> 32), cnt);
      cnt = __builtin_amdgcn_mbcnt_lo((uint32_t)O, cnt);
      cnt = __builtin_amdgcn_mbcnt_hi((uint32_t)(O >> 32), cnt);
      uint32_t base = s0 + m + cb * W - pc * pref_at(2u * q * kWaves, 2u);
      if constexpr (decltype(one_seg)::value) base = uniform(base);  // formed by scalar instructions
      const uint32_t pos = base + lane2w + __mul24(npc, (int)cnt);
      const uint32_t x = v2[q];
      uint32_t ext = 0;
      if constexpr (NR == 0) {
        for (uint32_t r = 0; r < p.runs.n; ++r) ext |= (x >> p.runs.shift[r]) & ((uint32_t)p.runs.pmask[r] * 0x10001u);
      } else {
#pragma unroll
        for (uint32_t r = 0; r < NR; ++r) ext |= (x >> p.runs.shift[r]) & ((uint32_t)p.runs.pmask[r] * 0x10001u);
      }
      const uint32_t a0 = h0 ? (ext & 0xFFFFu) : (x & 0xFFFFu), a1 = h1 ? (ext >> 16) : (x >> 16);
      const uint32_t field = a0 | (a1 << (h0 ? wpc : W));
      lds_or_bits(obuf, pos, field);  // lanes past the tile's end hold 0 (chunks read as 0, not matching)
    }
  };
  if constexpr (kPair) {
    // the pair words are opaque from here on, so the compiler takes the ballots again
    // instead of keeping 32 of them (or their per-lane flags) across the barriers
#pragma unroll
    for (uint32_t q = 0; q < kQP; ++q) asm volatile("" : "+v"(v2[q]));
    if ((a.S & 127u) == 0u) pair_passes(std::true_type{});
    else pair_passes(std::false_type{});
  }
  // the passes of half h of the tile (kHalves == 2: the tile's two halves of
  // kTile / 2 chunks are packed and stored one after the other through an image of
  // half the size, whose bit 0 is the half's first bit, tile image bit H)
  auto pack_form = [&](auto hc, uint32_t H, auto mc) __attribute__((always_inline)) {
  constexpr uint32_t qb = decltype(hc)::value * (kQ / kHalves), qe = qb + kQ / kHalves;
#pragma unroll
  for (uint32_t q = qb; q < (kPair ? 0u : qe); ++q) {
    const uint32_t blk = q * kWaves + wave;  // this wavefront's 64-chunk block
    const uint32_t cb = blk * kWave;                 // its first tile chunk
    if (cb >= nch) continue;                         // uniform
    const uint32_t cl = cb + lane;
    const bool valid = cl < nch;
    const uint64_t Bq = kRetake ? match_ballot(q) : B[q];
    const bool h = __builtin_amdgcn_inverse_ballot_w64(Bq);
    auto payload = [&]() -> T {
      if constexpr (kPos && W == 64) {
        // in 32-bit halves: the free bits of the low half come first
        if (!h) return v[q];
        const uint64_t F = ~mtab[ip[q]];
        const uint32_t Flo = (uint32_t)F, Fhi = (uint32_t)(F >> 32);
        uint64_t lo, hi;
        if constexpr (decltype(mc)::value) {
          lo = extract_runs<uint32_t>((uint32_t)v[q], Flo);
          hi = extract_runs<uint32_t>((uint32_t)((uint64_t)v[q] >> 32), Fhi);
        } else {
          lo = (uint32_t)v[q] & Flo;
          hi = (uint32_t)((uint64_t)v[q] >> 32) & Fhi;
        }
        return (T)(lo | (hi << __builtin_popcount(Flo)));
      } else if constexpr (kPos) {
        if (!h) return v[q];
        const uint32_t F = (uint32_t)(~mtab[ip[q]] & low_lanes(W));
        if constexpr (decltype(mc)::value) return (T)extract_runs<uint32_t>((uint32_t)v[q], F);
        else return (T)((uint32_t)v[q] & F);
      } else {
        return h ? extract_free<T, NR>(v[q], p.runs) : v[q];
      }
    };
    if constexpr (kMode == kModeLargeS) {
      // the block lies inside one segment: everything but the lane's own count is uniform
      if constexpr (kPos) {
        // position metadata: header written here, saved-bit prefixes read from LDS
        const uint32_t s0 = seg_start(cb);
        const uint32_t gs = uniform(pref[s0 >> 6]);
        const uint32_t m = min(a.S, nch - s0);
        const uint32_t segbase = s0 * (W + 1) - gs;
        if (lane == 0) lds_or_field(obuf, segbase + (cb - s0) - H, Bq);  // 64 header bits
        const uint32_t c_cl = uniform(pref[blk]) + svx[q];
        if (valid) lds_or_field(obuf, segbase + m + (cl - s0) * W - (c_cl - gs) - H, payload());
      } else {
        // chunk cl's payload bit: a scalar part, the lane's W l, less pc times the
        // compressed chunks of this block below the lane.  Lanes past the tile's end
        // hold payload 0 (their chunk reads as 0 and does not match), so they OR
        // nothing and their position is never used.
        const uint32_t s0 = seg_start(cb);
        const uint32_t m = min(a.S, nch - s0);
        const uint32_t k = s0 + m + cb * W - pc * pref_at(q * kWaves, 1u) - H;
        lds_or_bits(obuf, lane_bits + k - __umul24(pc, count_below(Bq)), payload());
      }
    } else if constexpr (kMode == kModeSmallS) {
      const uint32_t s0 = cb + (lane & ~(a.S - 1u));
      const uint32_t m = min(a.S, nch - min(s0, nch));
      if constexpr (kPos) {
        const uint32_t gs = cost(min(s0, nch - 1u));
        const uint32_t segbase = s0 * (W + 1) - gs;
        if (valid && i_lane == 0) lds_or_field(obuf, segbase - H, (uint32_t)((Bq >> lane) & low_lanes(m)));  // header
        const uint32_t c_cl = uniform(pref[blk]) + svx[q];
        if (valid) lds_or_field(obuf, segbase + m + i_lane * W - (c_cl - gs) - H, payload());
      } else {
        const uint32_t gs = pc * (pref_at(q * kWaves, 1u) + popc(Bq & seg_below));
        if (valid && i_lane == 0)
          lds_or_bits(obuf, s0 * (W + 1) - gs - H, (uint32_t)((Bq >> lane) & low_lanes(m)));
        const uint32_t pos = s0 + m + cl * W - __umul24(pc, pref_at(q * kWaves, 1u) + count_below(Bq)) - H;
        lds_or_bits(obuf, pos, payload());  // lanes past the tile's end hold 0
      }
    } else {
      if (valid) {
        const uint32_t s0 = seg_start(cl);
        const uint32_t i = cl - s0;
        const uint32_t gs = cost(s0);
        const uint32_t m = min(a.S, nch - s0);
        const uint32_t segbase = s0 * (W + 1) - gs;
        if (h) atomicOr(&obuf[(segbase + i) >> 5], 1u << ((segbase + i) & 31u));
        const uint32_t c_cl = kPos ? uniform(pref[blk]) + svx[q] : __umul24(pc, uniform(pref[blk]) + count_below(Bq));
        lds_or_field(obuf, segbase + m + i * W - (c_cl - gs), payload());
      }
    }
  }
  if constexpr (kMode == kModeLargeS && !kPos) {
    // the headers: lane q of each wavefront ORs in block q * kWaves + wave's
    // 64 participation bits
    const uint32_t blk = lane * kWaves + wave, cb = blk * kWave;
    if (lane >= qb && lane < qe && cb < nch) {
      const uint32_t s0 = seg_start(cb);
      const uint32_t sh = (blk & 1u) * 32u;
      const uint64_t hdr = kPair ? interleave32((uint32_t)(bal[blk & ~1u] >> sh), (uint32_t)(bal[blk | 1u] >> sh))
                                 : bal[blk];
      lds_or_bits(obuf, s0 * W + cb - pc * pref[s0 >> 6] - H, hdr);
    }
  }
  };
  // one copy of the passes per extraction form; multi is uniform
  auto pack = [&](auto hc, uint32_t H) __attribute__((always_inline)) {
    if constexpr (kPos) {
      if (multi) pack_form(hc, H, std::true_type{});
      else pack_form(hc, H, std::false_type{});
    } else {
      pack_form(hc, H, std::true_type{});
    }
  };
  // kHalves == 2: a tile whose whole image fits the half-size buffer (at most the
  // size of half a tile stored raw) is packed entirely before the look-back and
  // stored once
  const bool whole = agg <= (uint64_t)(kTile / 2) * (W + 1);
  if constexpr (kRetake) {
    // as in the pair form: the chunks are opaque from here on, so the ballots are
    // taken again when packing rather than kept across the barriers
#pragma unroll
    for (uint32_t q = 0; q < kQ; ++q) asm volatile("" : "+v"(v[q]));
  }
  pack(std::integral_constant<uint32_t, 0>{}, 0u);
  if constexpr (kHalves == 2) {
    if (whole) pack(std::integral_constant<uint32_t, 1>{}, 0u);
  }
  __syncthreads();

  // 5. the tile's start bit: decoupled look-back over the predecessors
  if (wave == 0) {
    bool timed_out = false;
    const uint64_t excl = t == 0 ? 0ull
                                 : lookback_finish(a.status, a.st_lg, a.control, a.err, t, (int64_t)t - 1, 0, agg,
                                                   a.wait_limit, lane, timed_out);
    if (lane == 0) {
      s_excl = excl;
      s_failed = timed_out ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint64_t excl = s_excl;
  // a tile that gave up waiting has no valid start bit: it stores no stream bits,
  // and its offsets become ~0, which no decoder accepts (the segments' bit ranges
  // fail their checks), so the stream is refused even without an error word
  if (s_failed != 0u) {
    for (uint32_t r = tid; r < nsegt; r += kThreads) a.off[k0 + r] = ~0ull;
    if (t == a.ntiles - 1 && tid == 0) a.off[a.nseg] = ~0ull;
    return;
  }

  // 6. segment offsets
  for (uint32_t r = tid; r < nsegt; r += kThreads)
    a.off[k0 + r] = excl + (uint64_t)r * a.S * (W + 1) - (uint64_t)cost(r * a.S);
  if (t == a.ntiles - 1 && tid == 0) a.off[a.nseg] = excl + agg;

  // 7. store image bits [0, nbits) at stream bit s_bit.  Output dword d is stream
  //    dword (s_bit >> 7) * 4 + d, so interior stores are 16-byte aligned; image bit
  //    j is output bit sh0 + j, sh0 = s_bit & 127.  The dword holding the first bit,
  //    when shared, is shared with the previous tile (hand-over word) or, head_in_tile,
  //    with the previous half of this tile, whose bits of it are `carry`: this half
  //    writes it.  The dword holding the last bit, when shared, is shared with the
  //    next tile (hand-over word) or, tail_in_tile, with the next half: its bits go to
  //    s_carry and the next half writes it.
  const bool last = t == a.ntiles - 1;
  auto store = [&](uint64_t s_bit, uint64_t nbits, bool head_in_tile, bool tail_in_tile, uint32_t carry) {
    const uint32_t sh0 = (uint32_t)(s_bit & 127u);
    const uint32_t dq = sh0 >> 5, sh = sh0 & 31u;
    const uint32_t img_end = (uint32_t)((nbits + 31) >> 5);  // image dwords holding the bits
    auto img = [&](int32_t i) -> uint32_t { return (i >= 0 && (uint32_t)i < img_end) ? obuf[i] : 0u; };
    auto out_dw = [&](uint32_t d) -> uint32_t {
      const int32_t i = (int32_t)d - (int32_t)dq;
      return sh ? (img(i) << sh) | (img(i - 1) >> (32u - sh)) : img(i);
    };
    const uint32_t first_d = dq;                                 // dword holding the first bit
    const uint32_t last_d = (uint32_t)((sh0 + nbits - 1) >> 5);  // dword holding the last bit
    const bool has_head = sh != 0u;
    const bool has_tail = ((sh0 + nbits) & 31u) != 0u;
    const bool hand_head = has_head && !head_in_tile, hand_tail = has_tail && !tail_in_tile && !last;
    const bool keep_tail = has_tail && tail_in_tile;
    const uint32_t lo = first_d + (has_head ? 1u : 0u);
    const uint32_t hi = last_d + 1u - ((hand_tail || keep_tail) ? 1u : 0u);  // [lo, hi) stored directly
    uint32_t *gdst = a.stream + ((s_bit >> 7) << 2);
    // the hand-over atomics go first, from two wavefronts, so that their round trips
    // overlap the interior stores; their results are used after those
    uint32_t mine_tail = 0, mine_head = 0;
    uint64_t old_tail = 0, old_head = 0;
    if (tid == 0 && hand_tail) {
      mine_tail = out_dw(last_d);
      old_tail = atomic_or_agent(&a.tails[t], kTailReady | mine_tail);
    }
    if (tid == kWave && hand_head) {
      mine_head = out_dw(first_d);
      old_head = atomic_or_agent(&a.tails[t - 1], kHeadReady | mine_head);
    }
    if (tid == 0 && keep_tail) s_carry = out_dw(last_d);
    if (tid == 0 && has_head && head_in_tile) gdst[first_d] = out_dw(first_d) | carry;
    const uint32_t a4 = min((lo + 3u) & ~3u, hi), e4 = max(hi & ~3u, a4);
    for (uint32_t d = lo + tid; d < a4; d += kThreads) gdst[d] = out_dw(d);
    // interior: output dwords [d, d + 4) are image bits from 32 d - sh0 on, i.e. from
    // bit t = 128 - sh0 of the eight image dwords [d - 4, d + 4) (two aligned 16-byte
    // LDS reads; the image is zero past its last bit and a4 >= 4 unless sh0 == 0)
    const uint32_t t_sh = 128u - sh0, jt = t_sh >> 5, st = t_sh & 31u;
    auto al = [&](uint32_t hi, uint32_t lo) -> uint32_t { return __builtin_amdgcn_alignbit(hi, lo, st); };
    for (uint32_t d = a4 + 4 * tid; d < e4; d += 4 * kThreads) {
      const uint4 A = *reinterpret_cast<const uint4 *>(obuf + ((max(d, 4u) - 4u) & ~3u));
      const uint4 C = *reinterpret_cast<const uint4 *>(obuf + d);
      uint4 o;
      switch (jt) {  // uniform
        case 0: o = make_uint4(al(A.y, A.x), al(A.z, A.y), al(A.w, A.z), al(C.x, A.w)); break;
        case 1: o = make_uint4(al(A.z, A.y), al(A.w, A.z), al(C.x, A.w), al(C.y, C.x)); break;
        case 2: o = make_uint4(al(A.w, A.z), al(C.x, A.w), al(C.y, C.x), al(C.z, C.y)); break;
        case 3: o = make_uint4(al(C.x, A.w), al(C.y, C.x), al(C.z, C.y), al(C.w, C.z)); break;
        default: o = C; break;  // sh0 == 0
      }
      store_nt16(gdst + d, o);
    }
    for (uint32_t d = e4 + tid; d < hi; d += kThreads) gdst[d] = out_dw(d);
    if (tid == 0 && hand_tail && (old_tail & kHeadReady)) gdst[last_d] = mine_tail | (uint32_t)old_tail;
    if (tid == kWave && hand_head && (old_head & kTailReady)) gdst[first_d] = mine_head | (uint32_t)old_head;
  };
  if constexpr (kHalves == 1) {
    store(excl, agg, false, false, 0u);
  } else if (whole) {
    store(excl, agg, false, false, 0u);
  } else {
    // a tile larger than the buffer holds more than kTile / 2 chunks, so it has two
    // halves; the first half's segments end at chunk kTile / 2
    const uint64_t agg0 = (uint64_t)(kTile / 2) * (W + 1) - (uint64_t)cost(kTile / 2);
    store(excl, agg0, false, true, 0u);
    __syncthreads();  // the first half's image has been read
    for (uint32_t d = 4 * tid; d < a.obuf_dw; d += 4 * kThreads)
      *reinterpret_cast<uint4 *>(obuf + d) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    pack(std::integral_constant<uint32_t, 1>{}, (uint32_t)agg0);
    __syncthreads();
    store(excl + agg0, agg - agg0, true, false, s_carry);
  }
}

__global__ void __launch_bounds__(kBlock) zero_kernel(uint64_t *p, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) p[i] = 0;
}

}  // namespace

static inline uint64_t host_min(uint64_t x, uint64_t y) { return x < y ? x : y; }

template <typename T, uint32_t M, uint32_t NR, bool kPos = false, bool kPair = false>
static hipError_t launch_encode_t(const EncodeArgs &a, const CodecParams &p, size_t shmem, hipStream_t s) {
  // two-half tiles: 32-bit chunks with one Mask, 64-bit chunks (enc_halves)
  if constexpr (sizeof(T) >= 4 && !kPair && M != kModeGeneral && !(kPos && sizeof(T) == 4)) {
    if (a.halves == 2) {
      if constexpr (sizeof(T) == 8 && !kPos) {
        if (a.big) {
          hipLaunchKernelGGL((encode_kernel<T, M, NR, false, false, 2, true>), dim3((uint32_t)a.ntiles),
                             dim3(enc_threads(false, 64, true)), shmem, s, a, p);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((encode_kernel<T, M, NR, kPos, false, 2>), dim3((uint32_t)a.ntiles),
                         dim3(enc_threads(kPos, sizeof(T) * 8)), shmem, s, a, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((encode_kernel<T, M, NR, kPos, kPair>), dim3((uint32_t)a.ntiles),
                     dim3(enc_threads(kPos, sizeof(T) * 8)), shmem, s, a, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_encode_pos_w(const EncodeArgs &a, const CodecParams &p, size_t shmem, hipStream_t s) {
  if (a.S % kWave == 0) return launch_encode_t<T, kModeLargeS, 0, true>(a, p, shmem, s);
  if (kWave % a.S == 0) return launch_encode_t<T, kModeSmallS, 0, true>(a, p, shmem, s);
  return launch_encode_t<T, kModeGeneral, 0, true>(a, p, shmem, s);
}

template <typename T, uint32_t M, bool kPair = false>
static hipError_t launch_encode_runs(const EncodeArgs &a, const CodecParams &p, size_t shmem, hipStream_t s) {
  switch (runs_bucket(p.runs.n)) {
    case 1: return launch_encode_t<T, M, 1, false, kPair>(a, p, shmem, s);
    case 2: return launch_encode_t<T, M, 2, false, kPair>(a, p, shmem, s);
    case 3: return launch_encode_t<T, M, 3, false, kPair>(a, p, shmem, s);
    case 4: return launch_encode_t<T, M, 4, false, kPair>(a, p, shmem, s);
    case 5: return launch_encode_t<T, M, 5, false, kPair>(a, p, shmem, s);
    case 6: return launch_encode_t<T, M, 6, false, kPair>(a, p, shmem, s);
    case 7: return launch_encode_t<T, M, 7, false, kPair>(a, p, shmem, s);
    case 8: return launch_encode_t<T, M, 8, false, kPair>(a, p, shmem, s);
    default: return launch_encode_t<T, M, 0, false, kPair>(a, p, shmem, s);
  }
}

template <typename T>
static hipError_t launch_encode_w(const EncodeArgs &a, const CodecParams &p, size_t shmem, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (a.pair) return launch_encode_runs<T, kModeLargeS, true>(a, p, shmem, s);
  }
  if (a.S % kWave == 0) return launch_encode_runs<T, kModeLargeS>(a, p, shmem, s);
  if (kWave % a.S == 0) return launch_encode_runs<T, kModeSmallS>(a, p, shmem, s);
  return launch_encode_t<T, kModeGeneral, 0>(a, p, shmem, s);
}

hipError_t launch_zero(uint64_t *p, uint64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint32_t blocks = (uint32_t)host_min((n + kBlock - 1) / kBlock, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(kBlock), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, const CodecParams &p, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  if (a.ntiles > 0x7FFFFFFFull) return hipErrorInvalidValue;
  // clear the control words, status and hand-over words (a kernel, not a
  // memset node, so the sequence stays valid inside a captured graph)
  hipError_t e = launch_zero(reinterpret_cast<uint64_t *>(a.control), 1 + status_words(a.ntiles) + a.ntiles, s);
  if (e != hipSuccess) return e;
  // image, ballots (kBal words), block prefixes (kBal + 1 words, padded to 8 bytes)
  const uint32_t tile = enc_tile_chunks(a.pmask != nullptr, a.pair != 0u, p.W, a.halves, a.big != 0u);
  size_t shmem = (size_t)a.obuf_dw * 4 + (tile / kWave) * 8 + ((tile / kWave) + 2) * 4;
  if (a.obuf_dw % 4 != 0) return hipErrorInvalidValue;
  if (a.pmask) {
    // position tables and per-chunk saved-bit prefixes (not for S a multiple of 64,
    // whose segments start on 64-chunk blocks)
    shmem += (size_t)a.S * 16 + (a.S % kWave == 0 ? 0 : (size_t)tile * 2);
    if (p.W == 16) return launch_encode_pos_w<uint16_t>(a, p, shmem, s);
    return p.W == 32 ? launch_encode_pos_w<uint32_t>(a, p, shmem, s) : launch_encode_pos_w<uint64_t>(a, p, shmem, s);
  }
  if (p.W == 16) return launch_encode_w<uint16_t>(a, p, shmem, s);
  return p.W == 32 ? launch_encode_w<uint32_t>(a, p, shmem, s) : launch_encode_w<uint64_t>(a, p, shmem, s);
}

}  // namespace ibp
