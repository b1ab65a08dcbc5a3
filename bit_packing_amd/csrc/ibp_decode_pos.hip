// ibp_decode_pos.hip -- step 3 of the IBP codec with position-dependent
// metadata, on gfx950: chunk position i of every segment has its own Mask_i and
// Bitval_i ("Riduzione del Collo di Bottiglia della Memoria GPU con la
// Compressione Lossless per il ML", section "Algoritmo Core", Preprocessing and
// Decompressione).  Contiguous stream in HBM, same stream layout as the
// single-Mask decoder.
//
// A matching chunk at position i keeps its bits outside Mask_i (the free
// positions F_i) packed low; decoding deposits them back into F_i and ORs in
// Bitval_i.  The free positions differ between lanes, so the deposit runs as
// log2(W) masked shift steps (the "expand" of H. S. Warren, Hacker's Delight,
// section 7-5): at step k, from the highest down, the positions in mv_k take the
// bit 2^k below them.  The masks mv_k depend on F_i alone; each workgroup
// computes them for every position into LDS once and then decodes tiles in a
// grid-stride loop, so that work is spread over many tiles.
//
// Per tile (as in the single-Mask decoder): check the segments' bit ranges and
// stage the tile's bits in LDS; per pass, a lane's payload offset is the
// segment's payload start plus the raw width of the chunks before it, minus the
// bits saved by the matching ones, popcount(Mask_j) each: an inclusive 64-lane
// scan of the savings.  Whole segments with S a multiple of 64 keep two running
// bit positions per segment; W <= 32 with S a multiple of 128 takes two chunks
// per lane (for W = 16 both go through the shift steps as one 32-bit word); any
// other S, and a short last segment, take the general loop with a per-segment
// carry in LDS.
#include <type_traits>

#include "ibp_decode_loops.h"

namespace ibp {
namespace {

using namespace dev;

// Threads per workgroup: W = 64 shares its larger position table (64 bytes per
// position) among 8 wavefronts, W <= 32 among 4 (measured on the 2^30-bf16 and
// integer-id workloads: 512 threads 10-15% faster at W = 64, 4-5% slower at W <= 32).
template <uint32_t W> constexpr uint32_t pos_block() { return W == 64 ? 512u : 256u; }

// (m & a) | (~m & b): one v_bfi_b32.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); }

// ------------------------------------------------------------------ position tables
//
// LDS layout: groups of four dwords (uint4), group-major, so that the lanes of a
// wavefront reading one group of consecutive positions read consecutive 16-byte
// words (no bank conflicts).  n = the entries per group.
//  W = 16: per pair of positions (2j, 2j + 1), n = ceil(S/2) pairs; group 0 =
//          mv_0 .. mv_3 as pair words (even position in the low half), group 1 =
//          F pair, Bitval pair, popcount(Mask) pair, 0.  Shift steps on a pair
//          word never carry across the halves: mv_k holds no position below 2^k
//          of either half.
//  W = 32: per position, even and odd positions apart, n = ceil(S/2): group
//          2g + (i & 1), entry i >> 1; group 0 = mv_0 .. mv_3, group 1 = mv_4, F,
//          Bitval, popcount(Mask).
//  W = 64: per position, n = S: group 0 = mv_0, mv_1 and group 1 = mv_2, mv_3
//          (low, high), group 2 = mv_4 (low, high), mv_5 high (its low half is
//          empty), 0; group 3 = F (low, high), Bitval (low, high).
// When no position needs a shift step (every F_i one run from bit 0: the packed
// bits already sit in place) the decoder reads only the group with F and Bitval.
template <uint32_t W> __host__ __device__ constexpr uint32_t pos_table_n(uint32_t S) {
  return W == 64 ? S : (S + 1u) / 2u;
}
template <uint32_t W> __host__ __device__ constexpr uint32_t pos_table_dw(uint32_t S) {
  return (W == 16 ? 8u : 16u) * pos_table_n<W>(S);
}

// mv_0 .. mv_{L-1} of the free-position mask F: the compress direction of the
// same steps, run on F itself.  At step k, mp marks the positions with an odd
// count of not-yet-moved gaps below them (a prefix XOR); the free positions
// among them move down by 2^k.
template <typename U, uint32_t L> __device__ __forceinline__ void expand_masks(U F, U (&mv)[L]) {
  U mk = (U)(~F << 1);
#pragma unroll
  for (uint32_t k = 0; k < L; ++k) {
    U mp = (U)(mk ^ (mk << 1));
#pragma unroll
    for (uint32_t s = 2; s < sizeof(U) * 8; s <<= 1) mp ^= (U)(mp << s);
    const U v = mp & F;
    mv[k] = v;
    F = (F ^ v) | (U)(v >> (1u << k));
    mk &= (U)~mp;
  }
}

// Returns a nonzero value when some position built by this thread needs a shift step.
template <uint32_t W>
__device__ __forceinline__ uint32_t build_pos_table(const uint64_t *pmask, const uint64_t *pbitval, uint32_t S,
                                                    uint4 *tab) {
  constexpr uint64_t kFull = W >= 64 ? ~0ull : ((1ull << W) - 1ull);
  const uint32_t n = pos_table_n<W>(S);
  uint32_t used = 0;
  if constexpr (W == 16) {
    for (uint32_t j = threadIdx.x; j < n; j += pos_block<W>()) {
      uint32_t w[7] = {0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (uint32_t h = 0; h < 2; ++h) {
        const uint32_t i = 2u * j + h;
        const uint32_t m = i < S ? (uint32_t)(pmask[i] & kFull) : (uint32_t)kFull;
        const uint32_t bv = i < S ? (uint32_t)(pbitval[i] & m) : 0u;
        uint32_t mv[4];
        expand_masks<uint32_t, 4>(~m & 0xFFFFu, mv);
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
          w[k] |= mv[k] << (16u * h);
          used |= mv[k];
        }
        w[4] |= (~m & 0xFFFFu) << (16u * h);
        w[5] |= bv << (16u * h);
        w[6] |= (uint32_t)__builtin_popcount(m) << (16u * h);
      }
      tab[j] = make_uint4(w[0], w[1], w[2], w[3]);
      tab[n + j] = make_uint4(w[4], w[5], w[6], 0u);
    }
  } else if constexpr (W == 32) {
    for (uint32_t i = threadIdx.x; i < S; i += pos_block<W>()) {
      const uint32_t m = (uint32_t)pmask[i];
      const uint32_t bv = (uint32_t)pbitval[i] & m;
      uint32_t mv[5];
      expand_masks<uint32_t, 5>(~m, mv);
      used |= mv[0] | mv[1] | mv[2] | mv[3] | mv[4];
      const uint32_t e = (i & 1u) * n + (i >> 1);
      tab[e] = make_uint4(mv[0], mv[1], mv[2], mv[3]);
      tab[2u * n + e] = make_uint4(mv[4], ~m, bv, (uint32_t)__builtin_popcount(m));
    }
  } else {
    for (uint32_t i = threadIdx.x; i < S; i += pos_block<W>()) {
      const uint64_t m = pmask[i];
      const uint64_t bv = pbitval[i] & m;
      uint64_t mv[6];
      expand_masks<uint64_t, 6>(~m, mv);
      const uint64_t any = mv[0] | mv[1] | mv[2] | mv[3] | mv[4] | mv[5];
      used |= (uint32_t)any | (uint32_t)(any >> 32);
      tab[i] = make_uint4((uint32_t)mv[0], (uint32_t)(mv[0] >> 32), (uint32_t)mv[1], (uint32_t)(mv[1] >> 32));
      tab[n + i] = make_uint4((uint32_t)mv[2], (uint32_t)(mv[2] >> 32), (uint32_t)mv[3], (uint32_t)(mv[3] >> 32));
      tab[2u * n + i] = make_uint4((uint32_t)mv[4], (uint32_t)(mv[4] >> 32), (uint32_t)(mv[5] >> 32), 0u);
      tab[3u * n + i] = make_uint4((uint32_t)~m, (uint32_t)(~m >> 32), (uint32_t)bv, (uint32_t)(bv >> 32));
    }
  }
  return used;
}

// ------------------------------------------------------------------ one position

// The shift steps of a W = 16 pair word y (either half may be junk when only the
// other is wanted), then F and Bitval: the decoded pair.
__device__ __forceinline__ uint32_t expand16x2(uint32_t y, const uint4 &e, const uint4 &f) {
  y = bfi(e.w, y << 8, y);
  y = bfi(e.z, y << 4, y);
  y = bfi(e.y, y << 2, y);
  y = bfi(e.x, y << 1, y);
  return bfi(f.x, y, f.y);
}

__device__ __forceinline__ uint32_t expand32(uint32_t y, const uint4 &e, const uint4 &f) {
  y = bfi(f.x, y << 16, y);
  y = bfi(e.w, y << 8, y);
  y = bfi(e.z, y << 4, y);
  y = bfi(e.y, y << 2, y);
  y = bfi(e.x, y << 1, y);
  return bfi(f.y, y, f.z);
}

// W = 64 in 32-bit halves: a shift by 2^k < 32 carries the top bits of the low
// half into the high half (alignbit); the shift by 32 moves the low half up.
__device__ __forceinline__ uint64_t expand64(uint64_t x, const uint4 &e0, const uint4 &e1, const uint4 &e2,
                                             const uint4 &e3) {
  uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  hi = bfi(e2.z, lo, hi);
  auto step = [&](uint32_t mlo, uint32_t mhi, uint32_t s) {
    const uint32_t th = __builtin_amdgcn_alignbit(hi, lo, 32u - s), tl = lo << s;
    hi = bfi(mhi, th, hi);
    lo = bfi(mlo, tl, lo);
  };
  step(e2.x, e2.y, 16);
  step(e1.z, e1.w, 8);
  step(e1.x, e1.y, 4);
  step(e0.z, e0.w, 2);
  step(e0.x, e0.y, 1);
  lo = bfi(e3.x, lo, e3.z);
  hi = bfi(e3.y, hi, e3.w);
  return ((uint64_t)hi << 32) | lo;
}

// W = 64: popcount(Mask) from F = (lo, hi).
__device__ __forceinline__ uint32_t pc64(const uint4 &f) {
  return 64u - (uint32_t)(__builtin_popcount(f.x) + __builtin_popcount(f.y));
}

// popcount(Mask_i) and the decoded value of a matching chunk at position i (n =
// entries per table group); kShift = false when no position needs a shift step.
template <typename T> __device__ __forceinline__ uint32_t pos_pc(const uint4 *tab, uint32_t n, uint32_t i) {
  constexpr uint32_t W = sizeof(T) * 8;
  if constexpr (W == 16) return (tab[n + (i >> 1)].z >> (16u * (i & 1u))) & 0xFFFFu;
  else if constexpr (W == 32) return tab[(2u + (i & 1u)) * n + (i >> 1)].w;
  else return pc64(tab[3u * n + i]);
}

template <typename T, bool kShift>
__device__ __forceinline__ T pos_apply(const uint4 *tab, uint32_t n, uint32_t i, T x) {
  constexpr uint32_t W = sizeof(T) * 8;
  if constexpr (W == 16) {
    const uint32_t sh = 16u * (i & 1u);
    const uint4 f = tab[n + (i >> 1)];
    if constexpr (!kShift) return (T)(bfi(f.x, (uint32_t)x << sh, f.y) >> sh);
    return (T)(expand16x2((uint32_t)x << sh, tab[i >> 1], f) >> sh);
  } else if constexpr (W == 32) {
    const uint32_t e = (i & 1u) * n + (i >> 1);
    const uint4 f = tab[2u * n + e];
    if constexpr (!kShift) return (T)bfi(f.y, (uint32_t)x, f.z);
    return (T)expand32((uint32_t)x, tab[e], f);
  } else {
    const uint4 f = tab[3u * n + i];
    if constexpr (!kShift)
      return (T)(((uint64_t)bfi(f.y, (uint32_t)((uint64_t)x >> 32), f.w) << 32) | bfi(f.x, (uint32_t)x, f.z));
    return (T)expand64((uint64_t)x, tab[i], tab[n + i], tab[2u * n + i], f);
  }
}

__device__ __forceinline__ uint32_t last_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// ------------------------------------------------------------------ whole segments

// One chunk per lane, S a multiple of 64: chunk q + lane of pass q.  hp is the
// header bit of the pass's first chunk, base its payload bit if every earlier
// chunk of the segment were raw.
template <typename T, bool kShift>
__device__ __forceinline__ uint32_t pos_row1(uint32_t S, const uint4 *tab, uint32_t n, const uint32_t *stg,
                                             uint32_t lb, uint32_t le, T *o, uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  if (lb == kBad) return 0u;
  o += lane;
  uint32_t hp = lb, base = lb + S;
  for (uint32_t q = 0; q < S; q += kWave) {
    const uint64_t H = uniform64(lds_field<uint64_t>(stg, hp));
    const bool h = __builtin_amdgcn_inverse_ballot_w64(H);
    const uint32_t s = h ? pos_pc<T>(tab, n, q + lane) : 0u;
    const uint32_t incl = wave_incl_scan(s);
    const T x = lds_field<T>(stg, base + lane * W - (incl - s));
    store_nt(&o[q], h ? pos_apply<T, kShift>(tab, n, q + lane, x) : x);
    base += kWave * W - last_lane(incl);
    hp += kWave;
  }
  return base != le ? IBP_DEVERR_CORRUPT : 0u;
}

// Two chunks per lane, W <= 32 and S a multiple of 128: lane l takes chunks 2l and
// 2l + 1 of each 128-chunk pass, reads their two participation bits, and stores
// them as one 2W-bit word (o aligned to 2W/8 bytes).
template <typename T, bool kShift>
__device__ __forceinline__ uint32_t pos_row2(uint32_t S, const uint4 *tab, uint32_t n, const uint32_t *stg,
                                             uint32_t lb, uint32_t le, T *o, uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  static_assert(W <= 32, "two chunks per lane up to W = 32");
  using P = typename std::conditional<(W == 32), uint64_t, uint32_t>::type;
  if (lb == kBad) return 0u;
  P *op = reinterpret_cast<P *>(o) + lane;
  uint32_t hp = lb + 2u * lane, base = lb + S;
  for (uint32_t q = 0; q < S; q += 2 * kWave) {
    const uint32_t b2 = lds_field<uint32_t>(stg, hp);
    const bool h0 = (b2 & 1u) != 0u, h1 = (b2 & 2u) != 0u;
    const uint32_t i = q + 2u * lane;
    if constexpr (W == 16) {
      const uint4 e1 = tab[n + (i >> 1)];  // the pair's groups: F, Bitval, popcounts; shift masks
      const uint32_t s0 = h0 ? (e1.z & 0xFFFFu) : 0u, s1 = h1 ? (e1.z >> 16) : 0u;
      const uint32_t s = s0 + s1;
      const uint32_t incl = wave_incl_scan(s);
      // both chunks lie in the 32 bits from chunk 2l's payload; the second sits
      // 16 - popcount(Mask) bits up when the first matches
      const uint32_t w = lds_field<uint32_t>(stg, base + 2u * lane * W - (incl - s));
      const uint32_t x = bfi(0xFFFFu, w, w << s0);
      const uint32_t sel = (h0 ? 0x0000FFFFu : 0u) | (h1 ? 0xFFFF0000u : 0u);
      store_nt(&op[q / 2], (P)bfi(sel, kShift ? expand16x2(x, tab[i >> 1], e1) : bfi(e1.x, x, e1.y), x));
      base += 2u * kWave * W - last_lane(incl);
    } else {
      const uint32_t j = i >> 1;  // positions i (even) and i + 1 (odd)
      const uint4 a1 = tab[2u * n + j], b1 = tab[3u * n + j];
      const uint32_t s0 = h0 ? a1.w : 0u, s1 = h1 ? b1.w : 0u;
      const uint32_t s = s0 + s1;
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t pos0 = base + 2u * lane * W - (incl - s), pos1 = pos0 + W - s0;
      const uint32_t x0 = lds_field<uint32_t>(stg, pos0), x1 = lds_field<uint32_t>(stg, pos1);
      uint32_t v0 = bfi(a1.y, x0, a1.z), v1 = bfi(b1.y, x1, b1.z);
      if constexpr (kShift) {
        v0 = expand32(x0, tab[j], a1);
        v1 = expand32(x1, tab[n + j], b1);
      }
      v0 = h0 ? v0 : x0;
      v1 = h1 ? v1 : x1;
      store_nt(&op[q / 2], (P)v0 | ((P)v1 << 32));
      base += 2u * kWave * W - last_lane(incl);
    }
    hp += 2u * kWave;
  }
  return base != le ? IBP_DEVERR_CORRUPT : 0u;
}

// Four chunks per lane, W = 16 and S a multiple of 256: lane l takes chunks 4l ..
// 4l + 3 of each 256-chunk pass (one savings scan per four chunks).  The four lie
// in the 64 bits from chunk 4l's payload bit, read once; chunk k + 1 starts 16 bits
// after chunk k, popcount(Mask) fewer when chunk k matches.  Chunks 4l, 4l + 1 and
// 4l + 2, 4l + 3 go through the shift steps as two pair words, stored as one
// 64-bit word (o 8-byte aligned).
template <bool kShift>
__device__ __forceinline__ uint32_t pos_row4(uint32_t S, const uint4 *tab, uint32_t n, const uint32_t *stg,
                                             uint32_t lb, uint32_t le, uint16_t *o, uint32_t lane) {
  constexpr uint32_t W = 16;
  if (lb == kBad) return 0u;
  uint64_t *op = reinterpret_cast<uint64_t *>(o) + lane;
  uint32_t hp = lb + 4u * lane, base = lb + S;
  for (uint32_t q = 0; q < S; q += 4 * kWave) {
    const uint32_t b4 = lds_field<uint32_t>(stg, hp);
    const bool h0 = (b4 & 1u) != 0u, h1 = (b4 & 2u) != 0u, h2 = (b4 & 4u) != 0u, h3 = (b4 & 8u) != 0u;
    const uint32_t j = q / 2u + 2u * lane;  // the lane's first pair of positions
    const uint4 fa = tab[n + j], fb = tab[n + j + 1u];  // F, Bitval, popcount pairs
    const uint32_t s0 = h0 ? (fa.z & 0xFFFFu) : 0u, s1 = h1 ? (fa.z >> 16) : 0u;
    const uint32_t s2 = h2 ? (fb.z & 0xFFFFu) : 0u, s3 = h3 ? (fb.z >> 16) : 0u;
    const uint32_t s = s0 + s1 + s2 + s3;
    const uint32_t incl = wave_incl_scan(s);
    const uint64_t w = lds_field<uint64_t>(stg, base + 4u * lane * W - (incl - s));
    const uint32_t o1 = W - s0, o2 = o1 + W - s1, o3 = o2 + W - s2;
    const uint32_t xa = ((uint32_t)w & 0xFFFFu) | ((uint32_t)(w >> o1) << 16);
    const uint32_t xb = ((uint32_t)(w >> o2) & 0xFFFFu) | ((uint32_t)(w >> o3) << 16);
    const uint32_t ya = kShift ? expand16x2(xa, tab[j], fa) : bfi(fa.x, xa, fa.y);
    const uint32_t yb = kShift ? expand16x2(xb, tab[j + 1u], fb) : bfi(fb.x, xb, fb.y);
    const uint32_t sa = (h0 ? 0x0000FFFFu : 0u) | (h1 ? 0xFFFF0000u : 0u);
    const uint32_t sb = (h2 ? 0x0000FFFFu : 0u) | (h3 ? 0xFFFF0000u : 0u);
    store_nt(&op[q / 4u], (uint64_t)bfi(sa, ya, xa) | ((uint64_t)bfi(sb, yb, xb) << 32));
    base += 4u * kWave * W - last_lane(incl);
    hp += 4u * kWave;
  }
  return base != le ? IBP_DEVERR_CORRUPT : 0u;
}

template <typename T, bool kShift>
__device__ __forceinline__ uint32_t pos_segment(uint32_t S, const uint4 *tab, uint32_t n, const uint32_t *stg,
                                                uint32_t lb, uint32_t le, T *o, uint32_t lane) {
  if constexpr (sizeof(T) == 2) {
    if (S % (4u * kWave) == 0u && (reinterpret_cast<uintptr_t>(o) & 7u) == 0u)
      return pos_row4<kShift>(S, tab, n, stg, lb, le, o, lane);
  }
  if constexpr (sizeof(T) <= 4) {
    if (S % (2u * kWave) == 0u && (reinterpret_cast<uintptr_t>(o) & (2u * sizeof(T) - 1u)) == 0u)
      return pos_row2<T, kShift>(S, tab, n, stg, lb, le, o, lane);
  }
  return pos_row1<T, kShift>(S, tab, n, stg, lb, le, o, lane);
}

// ------------------------------------------------------------------ S dividing 64

// S divides 64 and every segment of the tile is whole: a pass of 64 chunks holds
// 64/S whole segments, so a lane's saved bits are the wave scan less its value just
// before the segment's first lane (no segment continues into the next pass).
template <typename T, bool kShift>
__device__ __forceinline__ uint32_t pos_small(const DecodeArgs &a, const uint4 *tab, uint32_t n, const uint32_t *stg,
                                              const uint32_t *lbeg, const uint32_t *lend, uint32_t nch, T *out,
                                              uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  const uint32_t i = lane & (a.S - 1u);  // position in the segment
  const uint32_t first = lane - i;       // the segment's first lane
  uint32_t err = 0;
  for (uint32_t p0 = 0; p0 < nch; p0 += kWave) {
    const uint32_t cl = p0 + lane;
    const uint32_t lb = cl < nch ? lbeg[cl >> a.s_log2] : kBad;  // lanes past the tile: whole segments too
    const bool ok = lb != kBad;
    const bool h = ok && lds_bit(stg, lb + i);
    const uint32_t pci = ok ? pos_pc<T>(tab, n, i) : 0u;
    const uint32_t sv = h ? pci : 0u;
    const uint32_t x = wave_incl_scan(sv);
    const uint32_t xs = __shfl(x, first == 0u ? 0u : first - 1u, kWave);
    const uint32_t pos = ok ? lb + a.S + i * W - (x - sv - (first == 0u ? 0u : xs)) : 0u;
    const T xv = lds_field<T>(stg, pos);
    if (ok) {
      store_nt(&out[cl], h ? pos_apply<T, kShift>(tab, n, i, xv) : xv);
      if (i == a.S - 1u && pos + (h ? W - pci : W) != lend[cl >> a.s_log2]) err |= IBP_DEVERR_CORRUPT;
    }
  }
  return err;
}

// ------------------------------------------------------------------ any S

// Per pass of 64 tile chunks: the savings scan, less the part before the
// segment's first lane in the pass, plus the segment's carry from earlier passes.
template <typename T, bool kShift>
__device__ __forceinline__ uint32_t pos_general(const DecodeArgs &a, const uint4 *tab, uint32_t n, const uint32_t *stg,
                                                const uint32_t *lbeg, const uint32_t *lend, uint32_t *carry,
                                                uint32_t nu, uint32_t nch, T *out, uint32_t lane) {
  constexpr uint32_t W = sizeof(T) * 8;
  uint32_t err = 0;
  for (uint32_t r = lane; r < nu; r += kWave) carry[r] = 0;
  wave_lds_sync();
  for (uint32_t p0 = 0; p0 < nch; p0 += kWave) {
    const uint32_t cl = p0 + lane;
    const bool valid = cl < nch;
    const uint32_t r = valid ? (a.s_log2 != kNotPow2 ? cl >> a.s_log2 : cl / a.S) : 0u;
    const uint32_t i = cl - r * a.S;
    const uint32_t lb = valid ? lbeg[r] : kBad;
    const bool ok = lb != kBad;
    const uint32_t m = min(a.S, nch - r * a.S);
    const bool h = ok && lds_bit(stg, lb + i);
    const uint32_t pci = ok ? pos_pc<T>(tab, n, i) : 0u;
    const uint32_t sv = h ? pci : 0u;
    const uint32_t x = wave_incl_scan(sv);
    const uint32_t start = lane >= i ? lane - i : 0u;  // the segment's first lane in this pass
    const uint32_t xs = __shfl(x, start == 0u ? 0u : start - 1u, kWave);
    const uint32_t before = start == 0u ? 0u : xs;
    const uint32_t c = ok ? carry[r] : 0u;
    const uint32_t pos = ok ? lb + m + i * W - (c + x - sv - before) : 0u;
    const T xv = lds_field<T>(stg, pos);
    if (ok) {
      store_nt(&out[cl], h ? pos_apply<T, kShift>(tab, n, i, xv) : xv);
      if (i == m - 1 && pos + (h ? W - pci : W) != lend[r]) err |= IBP_DEVERR_CORRUPT;
    }
    wave_lds_sync();
    // the last lane of a segment that continues into the next pass keeps its carry
    if (ok && lane == kWave - 1 && i != m - 1) carry[r] = c + x - before;
    wave_lds_sync();
  }
  return err;
}

// ------------------------------------------------------------------ kernel

// kOcc8: registers bounded for 8 wavefronts per SIMD (the compiler otherwise takes
// about 106 scalar registers, which leaves room for 7, so 3 workgroups of 512 threads
// per CU); the host launches this form where it gives more resident workgroups.
template <typename T, bool kOcc8>
__global__ void __launch_bounds__(pos_block<sizeof(T) * 8>(), kOcc8 ? 8 : 1)
    decode_pos_kernel(DecodeArgs a, CodecParams p) {
  constexpr uint32_t W = sizeof(T) * 8;
  constexpr uint32_t kWaves = pos_block<W>() / kWave;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint4 *tab = reinterpret_cast<uint4 *>(smem);
  const uint32_t n = pos_table_n<W>(a.S);
  __shared__ uint32_t any_shift;
  if (threadIdx.x == 0) any_shift = 0;
  __syncthreads();
  if (build_pos_table<W>(a.pmask, a.pbitval, a.S, tab)) atomicOr(&any_shift, 1u);
  __syncthreads();
  const bool shift = uniform(any_shift) != 0u;
  const uint32_t lane = lane_id(), wave = uniform(threadIdx.x / kWave);
  uint32_t *stg = smem + pos_table_dw<W>(a.S) + (uint64_t)wave * a.wave_dw;
  uint32_t *lbeg = stg + a.stage_dw;
  uint32_t *lend = lbeg + a.G;
  uint32_t *carry = lend + a.G;  // saved bits of each segment in earlier passes
  const uint64_t ntiles = (a.n_units + a.G - 1u) / a.G;
  uint32_t err = 0;
  for (uint64_t t = (uint64_t)blockIdx.x * kWaves + wave; t < ntiles; t += (uint64_t)gridDim.x * kWaves) {
    const uint64_t u0 = t * a.G;
    const uint32_t nu = (uint32_t)min((uint64_t)a.G, a.n_units - u0);
    const uint64_t chunk0 = u0 * a.S;
    const uint32_t nch = (uint32_t)min((uint64_t)nu * a.S, a.n_chunks - chunk0);
    if (stage_tile<W>(a, u0, nu, nch, stg, lbeg, lend, lane, err)) {
      T *out = static_cast<T *>(a.out) + chunk0;
      wave_lds_sync();
      if (a.S % kWave == 0 && nch == nu * a.S) {
        for (uint32_t r = 0; r < nu; ++r) {
          const uint32_t lb = uniform(lbeg[r]), le = uniform(lend[r]);
          T *o = out + (uint64_t)r * a.S;
          err |= shift ? pos_segment<T, true>(a.S, tab, n, stg, lb, le, o, lane)
                       : pos_segment<T, false>(a.S, tab, n, stg, lb, le, o, lane);
        }
      } else if (kWave % a.S == 0 && nch == nu * a.S) {
        err |= shift ? pos_small<T, true>(a, tab, n, stg, lbeg, lend, nch, out, lane)
                     : pos_small<T, false>(a, tab, n, stg, lbeg, lend, nch, out, lane);
      } else {
        err |= shift ? pos_general<T, true>(a, tab, n, stg, lbeg, lend, carry, nu, nch, out, lane)
                     : pos_general<T, false>(a, tab, n, stg, lbeg, lend, carry, nu, nch, out, lane);
      }
    }
    wave_lds_sync();  // the next tile's staging overwrites this one's
  }
  if (err && a.err) atomicOr(a.err, err);
}

template <typename T> hipError_t launch(const DecodeArgs &a, const CodecParams &p, hipStream_t s) {
  constexpr uint32_t W = sizeof(T) * 8;
  constexpr uint32_t kPosBlock = pos_block<W>(), kPosWaves = kPosBlock / kWave;
  const size_t shmem = (size_t)pos_table_dw<W>(a.S) * 4 + (size_t)a.wave_dw * 4 * kPosWaves;
  // four times as many workgroups as fit on the device at once, each looping over
  // its share of the tiles (measured: 1x leaves the GNN-shaped W = 32 decode 25%
  // slower, from uneven ends; 4x costs four table builds per workgroup slot)
  // The 8-wavefront form where it fits more workgroups per CU (W >= 32; measured:
  // mixed feature rows 210 -> 182 us, GNN-shaped rows 218 -> 207 us; where the LDS
  // already bounds the workgroups, as for the llm tensor's 256 positions, its
  // spilled scalar registers cost 1%, and at W = 16 4%)
  int dev = 0, cus = 0, per_cu = 0, per_cu8 = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_pos_kernel<T, false>, (int)kPosBlock, shmem);
  if (e == hipSuccess && W >= 32)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu8, decode_pos_kernel<T, true>, (int)kPosBlock, shmem);
  if (e != hipSuccess) return e;
  const bool occ8 = per_cu8 > per_cu;
  if (occ8) per_cu = per_cu8;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const uint64_t tiles = (a.n_units + a.G - 1) / a.G;
  const uint64_t need = (tiles + kPosWaves - 1) / kPosWaves;
  const uint64_t fit = (uint64_t)cus * (uint64_t)per_cu;
  const dim3 grid((uint32_t)(need < 4 * fit ? need : 4 * fit));
  if (occ8) hipLaunchKernelGGL((decode_pos_kernel<T, true>), grid, dim3(kPosBlock), shmem, s, a, p);
  else hipLaunchKernelGGL((decode_pos_kernel<T, false>), grid, dim3(kPosBlock), shmem, s, a, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_pos(const DecodeArgs &a, const CodecParams &p, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  if (!a.pmask || !a.pbitval) return hipErrorInvalidValue;
  if (p.W == 16) return launch<uint16_t>(a, p, s);
  if (p.W == 32) return launch<uint32_t>(a, p, s);
  return launch<uint64_t>(a, p, s);
}

}  // namespace ibp
