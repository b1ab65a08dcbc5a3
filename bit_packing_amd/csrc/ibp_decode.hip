// ibp_decode.hip -- step 3 of the IBP codec on gfx950: decompression of a
// contiguous stream held in HBM, and of a gather of rows read straight from
// pinned host memory ("Riduzione del Collo di Bottiglia della Memoria GPU con la
// Compressione Lossless per il ML", section "Algoritmo Core", Decompressione, and
// section "Integrazione del Sistema", PCIe Transfer Compression).
//
// Each wavefront decodes one tile of G units (segments for the contiguous decode,
// rows for the gather):
//  a. read the units' bit ranges from the offset table and check them, so that
//     no read leaves the stream and no LDS write leaves the tile's staging area;
//  b. stage the compressed bits in LDS with 16-byte loads: the contiguous tile is
//     one range, all its loads issued before any LDS write; a gather stages each
//     row in its own slot, and when a row's blocks fit one load per lane each row
//     is staged and decoded as soon as its own load lands;
//  c. per pass of 64 chunks, find each lane's payload offset from the
//     participation bits: every chunk before it in its segment costs W bits,
//     minus popcount(Mask) for each compressed one, so the offset is a prefix
//     count of the participation bits (v_mbcnt over a 64-bit mask); read the
//     payload from LDS, deposit it into the free positions and OR in Bitval, or
//     take it raw; store 64 consecutive chunks.
// The prefix count has three forms, chosen by the host from S:
//  - S a multiple of 64: a pass lies inside one segment, whose 64 participation
//    bits are one broadcast 64-bit LDS read; for W <= 32 and S a multiple of 128
//    a lane takes two chunks of a 128-chunk pass instead (its own two
//    participation bits, the ballots of the even and the odd chunks), and for
//    W = 16 and S a multiple of 256 four chunks of a 256-chunk pass (four
//    ballots), and stores them as one word;
//  - S dividing 64: a pass holds 64/S whole segments; a ballot of the
//    participation bits, masked to the lane's segment;
//  - any other S: a ballot plus a per-segment carry kept in LDS.
#include <type_traits>

#include "ibp_decode_loops.h"

namespace ibp {
namespace {

using namespace dev;

template <typename T, bool kGather, uint32_t kMode, uint32_t NR>
__global__ void __launch_bounds__(kBlock, (kGather && sizeof(T) == 4) ? 8 : 1)
    decode_kernel(DecodeArgs a, CodecParams p) {
  constexpr uint32_t W = sizeof(T) * 8;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t lane = lane_id(), wave = uniform(threadIdx.x / kWave);
  const uint64_t u0 = ((uint64_t)blockIdx.x * kWavesPerBlock + wave) * a.G;
  if (u0 >= a.n_units) return;
  const uint32_t nu = (uint32_t)min((uint64_t)a.G, a.n_units - u0);
  uint32_t *stg = smem + (uint64_t)wave * a.wave_dw;
  uint32_t *lbeg = stg + a.stage_dw;
  uint32_t *lend = lbeg + a.G;
  uint32_t *gseg = lend + a.G;
  const uint64_t chunk0 = u0 * a.S;
  const uint32_t nch = (uint32_t)min((uint64_t)nu * a.S, a.n_chunks - chunk0);
  uint32_t err = 0;

  if constexpr (!kGather) {
    // a. the tile's range and its segments; b. stage
    if (!stage_tile<W>(a, u0, nu, nch, stg, lbeg, lend, lane, err)) return;
  } else {
    uint64_t *ufirst = reinterpret_cast<uint64_t *>(gseg + a.G + (a.G & 1u));
    uint32_t *unb = reinterpret_cast<uint32_t *>(ufirst + a.G);
    const uint64_t whole = a.stream_bytes >> 4;
    // a. rows; for S >= 64 (G <= 8) lane r also keeps row r's first block and its
    //    count of whole blocks in registers
    bool tail_row = false;
    uint64_t my_first = 0;
    uint32_t my_whole = 0;
    // checks and descriptors of row r from its id and bit range [x, y)
    auto describe = [&](uint32_t r, uint64_t x, uint64_t y, bool &good) {
      if (good && !(x <= y && y <= a.stream_bytes * 8u && y - x >= a.S && y - x <= (uint64_t)a.S * (W + 1))) {
        good = false;
        err |= IBP_DEVERR_CORRUPT;
      }
      const uint32_t slot = r * a.slot_dw * 32u;
      const uint64_t first = good ? x >> 7 : 0u;
      const uint32_t nb = good ? (uint32_t)(((y + 127u) >> 7) - first) : 0u;
      lbeg[r] = good ? slot + (uint32_t)(x & 127u) : kBad;
      lend[r] = good ? slot + (uint32_t)(y - (x & ~127ull)) : kBad;
      ufirst[r] = first;
      unb[r] = nb;
      tail_row |= good && first + nb > whole;
      return first;
    };
    for (uint32_t r = lane; r < nu; r += kWave) {
      const int64_t id = a.ids[u0 + r];
      bool good = id >= 0 && (uint64_t)id < a.nseg;
      if (!good) err |= IBP_DEVERR_BAD_ID;
      uint64_t x = 0, y = 0;
      if (good) {
        x = a.off[id];
        y = a.off[id + 1];
      }
      my_first = describe(r, x, y, good);
      my_whole = my_first >= whole ? 0u : (uint32_t)min((uint64_t)unb[r], whole - my_first);
    }
    wave_lds_sync();
    // b. stage every row into its slot: whole blocks first, all loads in flight
    //    before any LDS write
    if (a.S >= kWave && a.slot_dw <= 4u * kWave && whole > 0) {
      // a row's blocks fit one 16-byte load per lane: one load instruction per row
      // (row base address scalar).  A tile of one row (rows read over PCIe) issues
      // that one load.  Larger tiles issue all kGatherMaxRows loads unconditionally,
      // so the compiler can wait for each row's load alone.  Lanes past a row's
      // whole blocks re-read the row's last whole block (the same address as a
      // neighbouring lane, so no extra request); rows past the tile read block 0
      // of the stream.  Both write into the 16 spare bytes after the slots.
      static_assert(kGatherMaxRows == 8, "one named register per row");
      const uint32_t spare = a.G * a.slot_dw;
      auto fetch = [&](uint32_t r) -> uint4 {
        const uint32_t n_r = (uint32_t)__builtin_amdgcn_readlane((int)my_whole, (int)r);
        const uint64_t f_r = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_first >> 32), (int)r) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_first, (int)r);
        const uint64_t blk = min(f_r + min(lane, n_r ? n_r - 1u : 0u), whole - 1u);
        return *reinterpret_cast<const uint4 *>(a.stream + blk * 16u);
      };
      auto put = [&](uint32_t r, const uint4 &t) {
        const uint32_t n_r = (uint32_t)__builtin_amdgcn_readlane((int)my_whole, (int)r);
        *reinterpret_cast<uint4 *>(stg + (lane < n_r ? r * a.slot_dw + 4u * lane : spare)) = t;
      };
      if (a.G == 1) {
        // one row per wavefront (rows read over PCIe): one load, no other row
        const uint4 t0 = fetch(0);
        put(0, t0);
        if constexpr (kMode == kModeLargeS) {
          if (!ballot(tail_row)) {
            wave_lds_sync();
            err |= decode_segment<T, NR>(p, a.S, stg, uniform(lbeg[0]), uniform(lend[0]),
                                         static_cast<T *>(a.out) + chunk0, lane);
            if (err && a.err) atomicOr(a.err, err);
            return;
          }
        }
      } else {
      const uint4 t0 = fetch(0), t1 = fetch(1), t2 = fetch(2), t3 = fetch(3);
      const uint4 t4 = fetch(4), t5 = fetch(5), t6 = fetch(6), t7 = fetch(7);
      if constexpr (kMode == kModeLargeS) {
        if (!ballot(tail_row)) {
          // decode each row as soon as its own blocks have arrived, while the
          // later rows' loads are still in flight
          T *out = static_cast<T *>(a.out) + chunk0;
          // rows four at a time, their passes interleaved (four independent
          // LDS-latency chains)
          auto rows = [&](uint32_t r, const uint4 &t0, const uint4 &t1, const uint4 &t2, const uint4 &t3) {
            put(r, t0);
            put(r + 1, t1);
            put(r + 2, t2);
            put(r + 3, t3);
            wave_lds_sync();
            if (r + 3 < nu) {
              err |= decode_segments<T, NR, 4>(p, a.S, stg, lbeg, lend, r, out + (uint64_t)r * a.S, lane);
            } else {
              for (uint32_t k = r; k < nu; ++k)
                err |= decode_segment<T, NR>(p, a.S, stg, uniform(lbeg[k]), uniform(lend[k]), out + (uint64_t)k * a.S,
                                             lane);
            }
          };
          rows(0, t0, t1, t2, t3);
          rows(4, t4, t5, t6, t7);
          if (err && a.err) atomicOr(a.err, err);
          return;
        }
      }
      put(0, t0);
      put(1, t1);
      put(2, t2);
      put(3, t3);
      put(4, t4);
      put(5, t5);
      put(6, t6);
      put(7, t7);
      }
    } else if (a.S >= kWave) {
      // four loads in flight per lane before any LDS write
      // one load instruction per (row, 64 blocks): the row's base address is scalar
      uint32_t r = 0, j0 = 0;
      auto item = [&](uint4 &t, uint32_t &d) {
        d = kBad;
        if (r >= nu) return;
        const uint32_t n_r = (uint32_t)__builtin_amdgcn_readlane((int)my_whole, (int)r);
        const uint64_t f_r = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_first >> 32), (int)r) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_first, (int)r);
        const uint32_t j = j0 + lane;
        if (j < n_r) {
          t = *reinterpret_cast<const uint4 *>(a.stream + f_r * 16u + (j << 4));
          d = r * a.slot_dw + 4u * j;
        }
        j0 += kWave;
        if (j0 >= n_r) {
          j0 = 0;
          ++r;
        }
      };
      auto put = [&](const uint4 &t, uint32_t d) {
        if (d != kBad) *reinterpret_cast<uint4 *>(stg + d) = t;
      };
      while (r < nu) {
        uint4 t0, t1, t2, t3;
        uint32_t d0, d1, d2, d3;
        item(t0, d0);
        item(t1, d1);
        item(t2, d2);
        item(t3, d3);
        put(t0, d0);
        put(t1, d1);
        put(t2, d2);
        put(t3, d3);
      }
    } else {
      // flat over the rows' slot blocks; row = f / sb by a multiply-high with
      // sb_magic = ceil(2^32 / sb), exact for f, sb < 2^16
      const uint32_t sb = a.slot_dw / 4u;
      const uint32_t total = nu * sb;
      for (uint32_t f0 = 0; f0 < total; f0 += 4 * kWave) {
        uint4 tmp[4];
        uint32_t dst[4];
#pragma unroll
        for (uint32_t u = 0; u < 4; ++u) {
          const uint32_t f = f0 + u * kWave + lane;
          const uint32_t r = __umulhi(f, a.sb_magic), j = f - __umul24(r, sb);
          dst[u] = kBad;
          if (f < total && j < unb[r] && ufirst[r] + j < whole) {
            tmp[u] = load16(a.stream, ufirst[r] + j);
            dst[u] = r * a.slot_dw + 4u * j;
          }
        }
#pragma unroll
        for (uint32_t u = 0; u < 4; ++u)
          if (dst[u] != kBad) *reinterpret_cast<uint4 *>(stg + dst[u]) = tmp[u];
      }
    }
    // the row that ends in the stream's last, partial block
    if (ballot(tail_row)) {
      for (uint32_t r = 0; r < nu; ++r) {
        const uint32_t n_r = uniform(unb[r]);
        const uint64_t f_r = uniform64(ufirst[r]);
        if (n_r == 0 || f_r + n_r <= whole) continue;
        for (uint32_t j = lane; j < n_r; j += kWave)
          if (f_r + j >= whole)
            *reinterpret_cast<uint4 *>(stg + r * a.slot_dw + 4u * j) = load16_tail(a.stream, a.stream_bytes, f_r + j);
      }
    }
  }
  wave_lds_sync();

  // c. decode
  T *out = static_cast<T *>(a.out) + chunk0;
  if constexpr (kMode == kModeLargeS) {
    // gathered rows are whole segments, and so is every segment of a contiguous tile
    // but possibly the stream's last
    if (kGather || nch == nu * a.S)
      err |= decode_rows<T, NR>(a, p, stg, lbeg, lend, nu, out, lane);
    else
      err |= decode_large_s<T, NR>(a, p, stg, lbeg, lend, nu, nch, out, lane);
  } else if constexpr (kMode == kModeSmallS) {
    err |= decode_small_s<T, kGather, NR>(a, p, stg, lbeg, lend, nch, out, lane);
  } else {
    err |= decode_general<T, kGather>(a, p, stg, lbeg, lend, gseg, nch, out, lane);
  }
  if (err && a.err) atomicOr(a.err, err);
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
    store_nt16(reinterpret_cast<uint4 *>(a.out) + f, x);
  }
}

// ------------------------------------------------------------------ launch

struct Launch {
  dim3 grid;
  size_t shmem;
  hipStream_t s;
};

template <typename T, bool G, uint32_t M, uint32_t NR>
hipError_t go(const DecodeArgs &a, const CodecParams &p, const Launch &l) {
  hipLaunchKernelGGL((decode_kernel<T, G, M, NR>), l.grid, dim3(kBlock), l.shmem, l.s, a, p);
  return hipGetLastError();
}

template <typename T, bool G, uint32_t M>
hipError_t go_runs(const DecodeArgs &a, const CodecParams &p, const Launch &l) {
  switch (runs_bucket(p.runs.n)) {
    case 1: return go<T, G, M, 1>(a, p, l);
    case 2: return go<T, G, M, 2>(a, p, l);
    case 3: return go<T, G, M, 3>(a, p, l);
    case 4: return go<T, G, M, 4>(a, p, l);
    case 5: return go<T, G, M, 5>(a, p, l);
    case 6: return go<T, G, M, 6>(a, p, l);
    case 7: return go<T, G, M, 7>(a, p, l);
    case 8: return go<T, G, M, 8>(a, p, l);
    default: return go<T, G, M, 0>(a, p, l);
  }
}

template <typename T, bool G>
hipError_t go_mode(const DecodeArgs &a, const CodecParams &p, const Launch &l) {
  if (a.S % kWave == 0) return go_runs<T, G, kModeLargeS>(a, p, l);
  if (kWave % a.S == 0) return go_runs<T, G, kModeSmallS>(a, p, l);
  return go<T, G, kModeGeneral, 0>(a, p, l);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, const CodecParams &p, bool gather, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  const uint64_t tiles = (a.n_units + a.G - 1) / a.G;
  const uint64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  if (a.S % kWave != 0 && kWave % a.S == 0 && a.s_log2 == kNotPow2) return hipErrorInvalidValue;
  const Launch l{dim3((uint32_t)blocks), (size_t)a.wave_dw * 4 * kWavesPerBlock, s};
  if (p.W == 16) return gather ? go_mode<uint16_t, true>(a, p, l) : go_mode<uint16_t, false>(a, p, l);
  if (p.W == 32) return gather ? go_mode<uint32_t, true>(a, p, l) : go_mode<uint32_t, false>(a, p, l);
  return gather ? go_mode<uint64_t, true>(a, p, l) : go_mode<uint64_t, false>(a, p, l);
}

hipError_t launch_raw_gather(const RawGatherArgs &a, hipStream_t s) {
  const uint64_t total = a.n_ids * a.row_blocks;
  if (total == 0) return hipSuccess;
  const uint64_t want = (total + kBlock - 1) / kBlock;
  const uint32_t blocks = (uint32_t)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(raw_gather_kernel, dim3(blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace ibp
