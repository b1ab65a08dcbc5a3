// ibp_decode_loops.h -- the staging of a contiguous tile and the per-pass decode
// loops shared by the packed-stream decoders (ibp_decode.hip, ibp_decode_pos.hip)
// and the fixed-slot decoder (ibp_slots.hip).
//
// Each loop decodes the units (segments / rows) of one wavefront's tile whose
// bits are staged in LDS: unit r occupies local bits [lbeg[r], lend[r]) (kBad =
// skip), header first.  A lane's payload offset inside its unit is m + i*W
// minus popcount(Mask) for every compressed chunk before it; the loops compute
// that prefix count for S a multiple of 64 (one broadcast 64-bit header word per
// pass, or each lane's own participation bits and one ballot per chunk of a lane
// when a lane takes two or four chunks), S dividing 64 (a ballot masked to the lane's unit), or any S
// (a ballot plus a per-unit carry kept in gseg).  Whole segments can be decoded
// several at a time with their passes interleaved, which gives the scheduler
// independent LDS-latency chains.
#pragma once

#include <type_traits>

#include "ibp_device.h"

namespace ibp {
namespace dev {

constexpr uint32_t kBad = 0xFFFFFFFFu;

enum : uint32_t {
  kModeGeneral = 0,  // any S
  kModeSmallS = 1,   // 64 % S == 0: each pass holds 64/S whole segments
  kModeLargeS = 2,   // S % 64 == 0: each pass lies inside one segment
};

// Stage the 16-byte blocks [blk0, blk0 + nb) of src into LDS at dst.  Whole
// blocks are loaded four per lane before any is written (up to 256 loads in
// flight per wavefront); the block holding the end of a source whose length is
// not a multiple of 16 is read byte by byte afterwards.
__device__ __forceinline__ void stage_range(const uint8_t *src, uint64_t nbytes, uint64_t blk0, uint32_t nb,
                                            uint32_t *dst, uint32_t lane) {
  const uint64_t whole = nbytes >> 4;
  const uint32_t nf = blk0 >= whole ? 0u : (uint32_t)min((uint64_t)nb, whole - blk0);
  for (uint32_t j0 = 0; j0 < nf; j0 += 4 * kWave) {
    uint4 t[4];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
      const uint32_t j = j0 + u * kWave + lane;
      if (j < nf) t[u] = load16(src, blk0 + j);
    }
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
      const uint32_t j = j0 + u * kWave + lane;
      if (j < nf) *reinterpret_cast<uint4 *>(dst + 4 * j) = t[u];
    }
  }
  for (uint32_t j = nf + lane; j < nb; j += kWave)
    *reinterpret_cast<uint4 *>(dst + 4 * j) = load16_tail(src, nbytes, blk0 + j);
}

// Contiguous decode, steps a and b for the tile of segments [u0, u0 + nu): check
// its bit range and every segment's, fill lbeg/lend (kBad for a bad segment), and
// stage the range into LDS.  Returns false (after flagging the error) when the
// tile's range itself is unusable.
template <uint32_t W>
__device__ __forceinline__ bool stage_tile(const DecodeArgs &a, uint64_t u0, uint32_t nu, uint32_t nch, uint32_t *stg,
                                           uint32_t *lbeg, uint32_t *lend, uint32_t lane, uint32_t &err) {
  const uint64_t A = a.off[u0], B = a.off[u0 + nu];
  const bool tile_ok = A <= B && B - A <= (uint64_t)nch * (W + 1) && B <= a.stream_bytes * 8u;
  if (!tile_ok) {
    if (lane == 0 && a.err) atomicOr(a.err, IBP_DEVERR_CORRUPT);
    return false;
  }
  const uint64_t base = A & ~127ull;
  for (uint32_t r = lane; r < nu; r += kWave) {
    const uint64_t x = a.off[u0 + r], y = a.off[u0 + r + 1];
    const uint64_t m = min((uint64_t)a.S, a.n_chunks - (u0 + r) * a.S);
    const bool good = A <= x && x <= y && y <= B && y - x >= m && y - x <= m * (W + 1);
    lbeg[r] = good ? (uint32_t)(x - base) : kBad;
    lend[r] = good ? (uint32_t)(y - base) : kBad;
    if (!good) err |= IBP_DEVERR_CORRUPT;
  }
  stage_range(a.stream, a.stream_bytes, A >> 7, (uint32_t)(((B + 127u) >> 7) - (A >> 7)), stg, lane);
  return true;
}

// S a multiple of 64: the segments of the tile one after another, 64 chunks per pass.
template <typename T, uint32_t NR>
__device__ __forceinline__ uint32_t decode_large_s(const DecodeArgs &a, const CodecParams &p, const uint32_t *stg,
                                                   const uint32_t *lbeg, const uint32_t *lend, uint32_t nu,
                                                   uint32_t nch, T *out, uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  const uint32_t pc = p.pc;
  const T bitval = (T)p.bitval;
  const uint32_t lane_bits = lane * W;
  uint32_t err = 0;
  for (uint32_t r = 0; r < nu; ++r) {
    const uint32_t lb = uniform(lbeg[r]);
    if (lb == kBad) continue;
    const uint32_t c0 = r * a.S;
    const uint32_t m = min(a.S, nch - c0);
    uint32_t run = 0;  // compressed chunks of the segment before this pass
    T *o = out + c0;
    for (uint32_t q = 0; q < m; q += kWave) {
      uint64_t H = uniform64(lds_field<uint64_t>(stg, lb + q));  // this pass's participation bits
      const bool full = m - q >= kWave;
      if (!full) H &= low_lanes(m - q);
      // payload bit of chunk q + lane: the chunks before it in the segment cost W bits
      // each, pc fewer for every compressed one (the wave-uniform part is scalar)
      const uint32_t pos = (lb + m + q * W - pc * run) + lane_bits - __umul24(pc, count_below(H));
      const T x = lds_field<T>(stg, pos);
      const T v = __builtin_amdgcn_inverse_ballot_w64(H) ? (deposit_free<T, NR>(x, p.runs) | bitval) : x;
      if (full || lane < m - q) store_nt(&o[q + lane], v);
      run += popc(H);
    }
    if (lb + m + m * W - pc * run != uniform(lend[r])) err |= IBP_DEVERR_CORRUPT;
  }
  return err;
}

// A whole segment of S chunks (S a multiple of 64) whose bits are local bits
// [lb, le): every pass is full, so the per-pass bookkeeping reduces to two
// running bit positions: hp, the header bit of the pass's first chunk, and base,
// the payload bit it would have if every earlier chunk of the segment were raw.
template <typename T, uint32_t NR> struct Row1 {
  static constexpr uint32_t W = sizeof(T) * 8;
  static constexpr uint32_t kStep = kWave;  // chunks per pass
  uint32_t hp = 0, base = 0;
  T *o = nullptr;
  Row1() = default;
  __device__ __forceinline__ Row1(const CodecParams &, uint32_t S, uint32_t lb, T *out, uint32_t lane)
      : hp(lb), base(lb + S), o(out + lane) {}
  __device__ __forceinline__ void pass(const CodecParams &p, const uint32_t *stg, uint32_t q, uint32_t lane) {
    const uint64_t H = uniform64(lds_field<uint64_t>(stg, hp));  // this pass's participation bits
    const uint32_t pos = base + lane * W - __umul24(p.pc, count_below(H));
    const T x = lds_field<T>(stg, pos);
    store_nt(&o[q], __builtin_amdgcn_inverse_ballot_w64(H) ? (deposit_free<T, NR>(x, p.runs) | (T)p.bitval) : x);
    base += kWave * W - p.pc * popc(H);
    hp += kWave;
  }
};

// Two W = 16 chunks in one word x (chunk a in bits 0-15, b in 16-31, each
// payload from bit 0 of its half): deposit both with each run's mask in both
// halves (a run never crosses a half), OR in Bitval, and keep the raw half of a
// chunk that did not participate.
template <uint32_t NR>
__device__ __forceinline__ uint32_t merge16x2(const CodecParams &p, uint32_t x, bool ha, bool hb) {
  uint32_t d = (uint32_t)(uint16_t)p.bitval * 0x10001u;
  if constexpr (NR == 0) {
    for (uint32_t r = 0; r < p.runs.n; ++r) d |= (x & ((uint32_t)p.runs.pmask[r] * 0x10001u)) << p.runs.shift[r];
  } else {
#pragma unroll
    for (uint32_t r = 0; r < NR; ++r) d |= (x & ((uint32_t)p.runs.pmask[r] * 0x10001u)) << p.runs.shift[r];
  }
  const uint32_t sel = (ha ? 0x0000FFFFu : 0u) | (hb ? 0xFFFF0000u : 0u);
  return (sel & d) | (~sel & x);
}

// The same for W <= 32 and S a multiple of 128, two chunks per lane: lane l takes
// chunks 2l and 2l + 1 of each 128-chunk pass and reads their two participation
// bits itself; the compressed chunks before chunk 2l are those below lane l in
// the ballot of the even chunks plus those in the ballot of the odd ones, and
// the two ballots' popcounts give the pass's total.  The pair is stored as one
// 2W-bit word, so o must be 2W/8-byte aligned.  For W = 16 both chunks lie in
// the 32 bits from chunk 2l's payload, read once; the second sits 16 - pc bits up
// when the first is compressed, and the deposit runs on the pair word with each
// run's mask in both halves (a run never crosses a half).
template <typename T, uint32_t NR> struct Row2 {
  static constexpr uint32_t W = sizeof(T) * 8;
  static_assert(W <= 32, "two chunks per lane up to W = 32");
  static constexpr uint32_t kStep = 2 * kWave;
  using P = typename std::conditional<(W == 32), uint64_t, uint32_t>::type;  // a pair of chunks
  // hd, hsh: the dword and the bit in it of this lane's first participation bit (a
  // pass is 128 bits, so hsh is the same in every pass and hd moves by 4)
  uint32_t hd = 0, hsh = 0, base = 0;
  P *op = nullptr;
  Row2() = default;
  __device__ __forceinline__ Row2(const CodecParams &, uint32_t S, uint32_t lb, T *out, uint32_t lane)
      : hd((lb + 2u * lane) >> 5), hsh((lb + 2u * lane) & 31u), base(lb + S),
        op(reinterpret_cast<P *>(out) + lane) {}
  __device__ __forceinline__ void pass(const CodecParams &p, const uint32_t *stg, uint32_t q, uint32_t lane) {
    const uint32_t pc = p.pc;
    const uint32_t b2 = __builtin_amdgcn_alignbit(stg[hd + 1u], stg[hd], hsh);
    // the selects below take the ballots back (one compare per bit)
    const uint64_t E = ballot((b2 & 1u) != 0u), O = ballot((b2 & 2u) != 0u);
    const bool h0 = __builtin_amdgcn_inverse_ballot_w64(E), h1 = __builtin_amdgcn_inverse_ballot_w64(O);
    uint32_t below = __builtin_amdgcn_mbcnt_lo((uint32_t)E, 0u);
    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(E >> 32), below);
    below = __builtin_amdgcn_mbcnt_lo((uint32_t)O, below);
    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(O >> 32), below);
    const uint32_t pos0 = base + lane * 2u * W + __mul24(-(int32_t)pc, (int32_t)below);
    if constexpr (W == 16) {
      const uint32_t w = lds_field<uint32_t>(stg, pos0);
      const uint32_t x = (w & 0xFFFFu) | ((w << (h0 ? pc : 0u)) & 0xFFFF0000u);
      store_nt(&op[q / 2], (P)merge16x2<NR>(p, x, h0, h1));
    } else {
      const uint32_t pos1 = pos0 + (h0 ? W - pc : W);
      const T x0 = lds_field<T>(stg, pos0), x1 = lds_field<T>(stg, pos1);
      const T v0 = h0 ? (T)(deposit_free<T, NR>(x0, p.runs) | (T)p.bitval) : x0;
      const T v1 = h1 ? (T)(deposit_free<T, NR>(x1, p.runs) | (T)p.bitval) : x1;
      store_nt(&op[q / 2], (P)v0 | ((P)v1 << W));
    }
    base += 2u * kWave * W - pc * (popc(E) + popc(O));
    hd += 2u * kWave / 32u;
  }
};

// W = 16 and S a multiple of 256, four chunks per lane: lane l takes chunks
// 4l, ..., 4l + 3 of each 256-chunk pass and reads their four participation bits
// itself; the compressed chunks before chunk 4l are those below lane l in the
// four ballots (one per chunk of a lane), whose popcounts give the pass's total.
// The four payloads lie in the 64 bits from chunk 4l's payload, read once; each
// starts W - pc bits after a compressed predecessor and W bits after a raw one.
// They are aligned into two pair words, merged as in Row2, and stored as one
// 8-byte word, so o must be 8-byte aligned.  Per chunk this halves the header,
// prefix-count and address work of Row2.
template <typename T, uint32_t NR> struct Row4 {
  static_assert(sizeof(T) == 2, "four chunks per lane for W = 16");
  static constexpr uint32_t W = 16;
  static constexpr uint32_t kStep = 4 * kWave;
  // hd, hsh: the dword and the bit in it of this lane's first participation bit (a
  // pass is 256 bits, so hsh is the same in every pass and hd moves by 8); lw: 4 W
  // times the lane; wpc: W - popcount(Mask), a compressed chunk's payload.  The
  // per-lane terms are opaque to the compiler, so they stay in vector registers
  // rather than being formed again from scalar values in every pass.
  uint32_t hd = 0, hsh = 0, base = 0, lw = 0, wpc = 0;
  uint64_t *op = nullptr;
  Row4() = default;
  __device__ __forceinline__ Row4(const CodecParams &p, uint32_t S, uint32_t lb, T *out, uint32_t lane)
      : base(lb + S), lw(lane * 4u * W), wpc(W - p.pc), op(reinterpret_cast<uint64_t *>(out) + lane) {
    const uint32_t hp = lb + 4u * lane;
    hd = hp >> 5;
    hsh = hp & 31u;
    asm volatile("" : "+v"(hd), "+v"(hsh), "+v"(lw), "+v"(wpc));
  }
  __device__ __forceinline__ void pass(const CodecParams &p, const uint32_t *stg, uint32_t q, uint32_t lane) {
    const uint32_t pc = p.pc;
    const uint32_t b4 = __builtin_amdgcn_alignbit(stg[hd + 1u], stg[hd], hsh);
    // the selects below take the ballots back (one compare per bit)
    const uint64_t B0 = ballot((b4 & 1u) != 0u), B1 = ballot((b4 & 2u) != 0u);
    const uint64_t B2 = ballot((b4 & 4u) != 0u), B3 = ballot((b4 & 8u) != 0u);
    const bool h0 = __builtin_amdgcn_inverse_ballot_w64(B0), h1 = __builtin_amdgcn_inverse_ballot_w64(B1);
    const bool h2 = __builtin_amdgcn_inverse_ballot_w64(B2), h3 = __builtin_amdgcn_inverse_ballot_w64(B3);
    // compressed chunks before chunk 4 lane: one chain of the lane-count instructions
    uint32_t below = __builtin_amdgcn_mbcnt_lo((uint32_t)B0, 0u);
    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(B0 >> 32), below);
    below = __builtin_amdgcn_mbcnt_lo((uint32_t)B1, below);
    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(B1 >> 32), below);
    below = __builtin_amdgcn_mbcnt_lo((uint32_t)B2, below);
    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(B2 >> 32), below);
    below = __builtin_amdgcn_mbcnt_lo((uint32_t)B3, below);
    below = __builtin_amdgcn_mbcnt_hi((uint32_t)(B3 >> 32), below);
    const uint64_t w = lds_field<uint64_t>(stg, (base + lw) + __mul24(-(int32_t)pc, (int32_t)below));
    const uint32_t o1 = h0 ? wpc : W, o2 = o1 + (h1 ? wpc : W), o3 = o2 + (h2 ? wpc : W);
    const uint32_t xa = ((uint32_t)w & 0xFFFFu) | ((uint32_t)(w >> o1) << 16);
    const uint32_t xb = ((uint32_t)(w >> o2) & 0xFFFFu) | ((uint32_t)(w >> o3) << 16);
    store_nt(&op[q / 4], (uint64_t)merge16x2<NR>(p, xa, h0, h1) | ((uint64_t)merge16x2<NR>(p, xb, h2, h3) << 32));
    base += 4u * kWave * W - pc * (popc(B0) + popc(B1) + popc(B2) + popc(B3));
    hd += 4u * kWave / 32u;
  }
};

template <typename R, typename T>
__device__ __forceinline__ uint32_t decode_one(const CodecParams &p, uint32_t S, const uint32_t *stg, uint32_t lb,
                                               uint32_t le, T *o, uint32_t lane) {
  if (lb == kBad) return 0u;
  R r(p, S, lb, o, lane);
  for (uint32_t q = 0; q < S; q += R::kStep) r.pass(p, stg, q, lane);
  return r.base != le ? IBP_DEVERR_CORRUPT : 0u;
}

// Chunks per lane for whole segments of S chunks (S a multiple of 64) stored from
// o: four for W = 16 with S a multiple of 256, two for W <= 32 with S a multiple
// of 128, the output aligned for the lane's word; else one.
template <typename T>
__device__ __forceinline__ uint32_t chunks_per_lane(uint32_t S, const T *o) {
  const uintptr_t ad = reinterpret_cast<uintptr_t>(o);
  if (sizeof(T) == 2 && S % (4u * kWave) == 0u && (ad & 7u) == 0u) return 4u;
  if (sizeof(T) <= 4 && S % (2u * kWave) == 0u && (ad & (2u * sizeof(T) - 1u)) == 0u) return 2u;
  return 1u;
}

// One whole segment.
template <typename T, uint32_t NR>
__device__ __forceinline__ uint32_t decode_segment(const CodecParams &p, uint32_t S, const uint32_t *stg, uint32_t lb,
                                                   uint32_t le, T *o, uint32_t lane) {
  const uint32_t per = chunks_per_lane(S, o);
  if constexpr (sizeof(T) == 2) {
    if (per == 4u) return decode_one<Row4<T, NR>, T>(p, S, stg, lb, le, o, lane);
  }
  if constexpr (sizeof(T) <= 4) {
    if (per == 2u) return decode_one<Row2<T, NR>, T>(p, S, stg, lb, le, o, lane);
  }
  return decode_one<Row1<T, NR>, T>(p, S, stg, lb, le, o, lane);
}

// K whole segments (rows) r, ..., r + K - 1 of S chunks each, S a multiple of 64,
// whose outputs follow each other from o: their passes are interleaved, K
// independent LDS-latency chains per step, when all are valid and take the same
// form; otherwise one at a time.
template <typename R, typename T, uint32_t K>
__device__ __forceinline__ uint32_t decode_interleaved(const CodecParams &p, uint32_t S, const uint32_t *stg,
                                                       const uint32_t (&lb)[K], const uint32_t (&le)[K], T *o,
                                                       uint32_t lane) {
  R rows[K] = {};
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) rows[k] = R(p, S, lb[k], o + (uint64_t)k * S, lane);
  for (uint32_t q = 0; q < S; q += R::kStep) {
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) rows[k].pass(p, stg, q, lane);
  }
  bool bad = false;
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) bad |= rows[k].base != le[k];
  return bad ? IBP_DEVERR_CORRUPT : 0u;
}

template <typename T, uint32_t NR, uint32_t K>
__device__ __forceinline__ uint32_t decode_segments(const CodecParams &p, uint32_t S, const uint32_t *stg,
                                                    const uint32_t *lbeg, const uint32_t *lend, uint32_t r, T *o,
                                                    uint32_t lane) {
  uint32_t lb[K], le[K];
  bool ok = true;
#pragma unroll
  for (uint32_t k = 0; k < K; ++k) {
    lb[k] = uniform(lbeg[r + k]);
    le[k] = uniform(lend[r + k]);
    ok &= lb[k] != kBad;
  }
  if (!ok) {
    uint32_t err = 0;
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) err |= decode_segment<T, NR>(p, S, stg, lb[k], le[k], o + (uint64_t)k * S, lane);
    return err;
  }
  const uint32_t per = chunks_per_lane(S, o);
  if constexpr (sizeof(T) == 2) {
    if (per == 4u) return decode_interleaved<Row4<T, NR>, T, K>(p, S, stg, lb, le, o, lane);
  }
  if constexpr (sizeof(T) <= 4) {
    if (per == 2u) return decode_interleaved<Row2<T, NR>, T, K>(p, S, stg, lb, le, o, lane);
  }
  return decode_interleaved<Row1<T, NR>, T, K>(p, S, stg, lb, le, o, lane);
}

// Units that are all whole segments of S chunks, S a multiple of 64, two at a time.
template <typename T, uint32_t NR>
__device__ __forceinline__ uint32_t decode_rows(const DecodeArgs &a, const CodecParams &p, const uint32_t *stg,
                                                const uint32_t *lbeg, const uint32_t *lend, uint32_t nu, T *out,
                                                uint32_t lane) {
  uint32_t err = 0;
  uint32_t r = 0;
  for (; r + 1 < nu; r += 2)
    err |= decode_segments<T, NR, 2>(p, a.S, stg, lbeg, lend, r, out + (uint64_t)r * a.S, lane);
  if (r < nu)
    err |= decode_segment<T, NR>(p, a.S, stg, uniform(lbeg[r]), uniform(lend[r]), out + (uint64_t)r * a.S, lane);
  return err;
}

// S dividing 64: each pass holds 64/S whole segments.
template <typename T, bool kGather, uint32_t NR>
__device__ __forceinline__ uint32_t decode_small_s(const DecodeArgs &a, const CodecParams &p, const uint32_t *stg,
                                                   const uint32_t *lbeg, const uint32_t *lend, uint32_t nch,
                                                   T *out, uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  const uint32_t pc = p.pc;
  const T bitval = (T)p.bitval;
  const uint32_t i = lane & (a.S - 1u);
  const uint64_t seg_below = low_lanes(lane & ~(a.S - 1u));  // lanes of earlier segments in the pass
  uint32_t err = 0;
  for (uint32_t p0 = 0; p0 < nch; p0 += kWave) {
    const uint32_t cl = p0 + lane;
    const bool valid = cl < nch;
    const uint32_t r = cl >> a.s_log2;
    const uint32_t lb = valid ? lbeg[r] : kBad;
    const bool ok = lb != kBad;
    uint32_t m = a.S;
    if constexpr (!kGather) m = valid ? min(a.S, nch - (r << a.s_log2)) : a.S;
    const bool h = ok && lds_bit(stg, lb + i);
    const uint64_t H = ballot(h);
    const uint32_t cnt = count_below(H) - popc(H & seg_below);
    const uint32_t pos = ok ? lb + m + i * W - pc * cnt : 0u;
    const T x = lds_field<T>(stg, pos);
    const T v = h ? (deposit_free<T, NR>(x, p.runs) | bitval) : x;
    if (ok) {
      store_nt(&out[cl], v);
      if (i == m - 1 && pos + (h ? W - pc : W) != lend[r]) err |= IBP_DEVERR_CORRUPT;
    }
  }
  return err;
}

// Any S: a segment may start anywhere in a pass and span passes; the number of
// compressed chunks before each segment start is kept in gseg.
template <typename T, bool kGather>
__device__ __forceinline__ uint32_t decode_general(const DecodeArgs &a, const CodecParams &p, const uint32_t *stg,
                                                   const uint32_t *lbeg, const uint32_t *lend, uint32_t *gseg,
                                                   uint32_t nch, T *out, uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  const uint32_t pc = p.pc;
  const T bitval = (T)p.bitval;
  uint32_t err = 0;
  uint32_t running = 0;  // compressed chunks among tile chunks [0, p0)
  for (uint32_t p0 = 0; p0 < nch; p0 += kWave) {
    const uint32_t cl = p0 + lane;
    const bool valid = cl < nch;
    const uint32_t r = cl / a.S;
    const uint32_t i = cl - r * a.S;
    const uint32_t lb = valid ? lbeg[r] : kBad;
    const bool ok = lb != kBad;
    uint32_t m = a.S;
    if constexpr (!kGather) m = valid ? min(a.S, nch - r * a.S) : a.S;
    const bool h = ok && lds_bit(stg, lb + i);
    const uint64_t H = ballot(h);
    const uint32_t g_cl = running + count_below(H);
    const uint32_t s0 = r * a.S;
    uint32_t g_start;
    if (s0 >= p0)
      g_start = running + popc(H & low_lanes(s0 - p0));
    else
      g_start = valid ? gseg[r] : 0u;
    if (valid && i == 0) gseg[r] = g_cl;
    const uint32_t pos = ok ? lb + m + i * W - pc * (g_cl - g_start) : 0u;
    const T x = lds_field<T>(stg, pos);
    const T v = h ? (deposit_free<T, 0>(x, p.runs) | bitval) : x;
    if (ok) {
      store_nt(&out[cl], v);
      if (i == m - 1 && pos + (h ? W - pc : W) != lend[r]) err |= IBP_DEVERR_CORRUPT;
    }
    running += popc(H);
    wave_lds_sync();
  }
  return err;
}

}  // namespace dev
}  // namespace ibp
