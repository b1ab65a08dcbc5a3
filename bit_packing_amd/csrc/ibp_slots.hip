// ibp_slots.hip -- the fixed-slot (in-place) layout of the IBP page's PCIe
// transfer compression ("Riduzione del Collo di Bottiglia della Memoria GPU con la
// Compressione Lossless per il ML", section "Integrazione del Sistema"): every
// row keeps a fixed slot of its raw size in (usually pinned host) memory, only the
// used part of a slot is read, and a bit vector in GPU memory says which rows are
// stored compressed.
//
// A row that compresses stores its segment bits (S participation bits, then the
// payloads, exactly as a segment of the packed stream) from bit 0 of its slot; a
// row that would not get shorter is stored raw.  The used length of a compressed
// slot is not stored: it follows from its header.
#include "ibp_decode_loops.h"

namespace ibp {
namespace {

using namespace dev;

// Compression: one wavefront per tile of G rows.  The rows' images are built in
// LDS (one region of img_dw dwords per row), then each row is stored compressed
// or raw into its slot, and its flag bit is set.
template <typename T, uint32_t NR>
__global__ void __launch_bounds__(kBlock) encode_slots_kernel(SlotArgs a, CodecParams p) {
  constexpr uint32_t W = sizeof(T) * 8;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t lane = lane_id(), wave = uniform(threadIdx.x / kWave);
  const uint64_t u0 = ((uint64_t)blockIdx.x * kWavesPerBlock + wave) * a.G;
  if (u0 >= a.n_units) return;
  const uint32_t nu = (uint32_t)min((uint64_t)a.G, a.n_units - u0);
  uint32_t *img = smem + (uint64_t)wave * a.wave_dw;
  uint32_t *gseg = img + a.G * a.img_dw;  // compressed chunks before each row start (nu + 1)
  for (uint32_t d = 4 * lane; d < nu * a.img_dw; d += 4 * kWave)
    *reinterpret_cast<uint4 *>(img + d) = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_sync();

  const T *in = static_cast<const T *>(a.in) + u0 * a.S;
  const uint32_t nch = nu * a.S;
  const T mask = (T)p.mask, bitval = (T)p.bitval;
  const uint32_t pc = p.pc;
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
    const T v = valid ? in[cl] : (T)0;
    const bool h = valid && ((v ^ bitval) & mask) == 0;
    const uint64_t H = ballot(h);
    const uint32_t g_cl = running + count_below(H);
    const uint32_t s0 = r * a.S;
    uint32_t g_start = 0;
    if (s0 >= p0)
      g_start = running + popc(H & low_lanes(s0 - p0));
    else if (valid)
      g_start = gseg[r];
    if (valid && i == 0) gseg[r] = g_cl;
    if (valid) {
      const uint32_t base = r * a.img_dw * 32u;
      if (h) atomicOr(&img[(base + i) >> 5], 1u << ((base + i) & 31u));
      const uint32_t pos = base + a.S + i * W - pc * (g_cl - g_start);
      lds_or_field(img, pos, h ? extract_free<T, NR>(v, p.runs) : v);
    }
    running += popc(H);
    wave_lds_sync();
  }
  if (lane == 0) gseg[nu] = running;
  wave_lds_sync();

  const uint32_t row_bits = a.row_bytes * 8u;
  const uint32_t row_q = a.row_bytes / 16u;
  for (uint32_t r = 0; r < nu; ++r) {
    const uint64_t row = u0 + r;
    const uint32_t matched = uniform(gseg[r + 1]) - uniform(gseg[r]);
    const uint32_t bits = a.S * (W + 1) - pc * matched;
    uint4 *dst = reinterpret_cast<uint4 *>(a.slots + row * a.row_bytes);
    if (bits < row_bits) {
      const uint32_t nq = (bits + 127u) / 128u;  // <= row_q because row_bytes % 16 == 0
      const uint4 *srcq = reinterpret_cast<const uint4 *>(img + r * a.img_dw);
      for (uint32_t q = lane; q < nq; q += kWave) dst[q] = srcq[q];
      if (lane == 0) atomicOr(reinterpret_cast<unsigned long long *>(&a.flags[row >> 6]), 1ull << (row & 63u));
    } else {
      const uint4 *srcq = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.in) + row * a.row_bytes);
      for (uint32_t q = lane; q < row_q; q += kWave) dst[q] = srcq[q];
    }
  }
}

// Gather: one wavefront per tile of G output rows.
//  a. each row's id, its flag, and its slot;
//  b. stage the first head_blocks 16-byte blocks of every slot (the header of a
//     compressed row; all of a raw row is staged);
//  c. a compressed row's length follows from its header; stage the rest of it;
//  d. raw rows are copied out, compressed rows go through the decode loops.
template <typename T, uint32_t kMode, uint32_t NR>
__global__ void __launch_bounds__(kBlock) decode_slots_kernel(SlotArgs a, CodecParams p) {
  constexpr uint32_t W = sizeof(T) * 8;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t lane = lane_id(), wave = uniform(threadIdx.x / kWave);
  const uint64_t u0 = ((uint64_t)blockIdx.x * kWavesPerBlock + wave) * a.G;
  if (u0 >= a.n_units) return;
  const uint32_t nu = (uint32_t)min((uint64_t)a.G, a.n_units - u0);
  uint32_t *stg = smem + (uint64_t)wave * a.wave_dw;
  uint32_t *lbeg = stg + a.G * a.img_dw;
  uint32_t *lend = lbeg + a.G;
  uint32_t *gseg = lend + a.G;
  uint32_t *kind = gseg + a.G;     // 0 = bad id, 1 = compressed, 2 = raw
  uint32_t *nblk = kind + a.G;     // blocks to stage
  uint32_t *nhead = nblk + a.G;    // blocks staged in the first round
  uint64_t *slot0 = reinterpret_cast<uint64_t *>(nhead + a.G + (a.G & 1u));  // first block of each slot
  const uint32_t row_blocks = a.row_bytes / 16u;
  uint32_t err = 0;

  // a.
  for (uint32_t r = lane; r < nu; r += kWave) {
    const int64_t id = a.ids[u0 + r];
    const bool good = id >= 0 && (uint64_t)id < a.n_rows;
    if (!good) err |= IBP_DEVERR_BAD_ID;
    const bool comp = good && ((a.flags[(uint64_t)id >> 6] >> ((uint64_t)id & 63u)) & 1ull);
    kind[r] = !good ? 0u : (comp ? 1u : 2u);
    slot0[r] = good ? (uint64_t)id * row_blocks : 0;
    nhead[r] = !good ? 0u : (comp ? min(a.head_blocks, row_blocks) : row_blocks);
  }
  wave_lds_sync();
  // b. first round of loads: the header blocks (or the whole raw row)
  const uint32_t total = nu * row_blocks;
  for (uint32_t f0 = 0; f0 < total; f0 += 4 * kWave) {
    uint4 tmp[4];
    uint32_t dst[4];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
      const uint32_t f = f0 + u * kWave + lane;
      const uint32_t r = f / row_blocks, j = f - r * row_blocks;
      dst[u] = kBad;
      if (f < total && j < nhead[r]) {
        tmp[u] = load16(a.slots, slot0[r] + j);
        dst[u] = r * a.img_dw + 4u * j;
      }
    }
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u)
      if (dst[u] != kBad) *reinterpret_cast<uint4 *>(stg + dst[u]) = tmp[u];
  }
  wave_lds_sync();
  // c. lengths of the compressed rows from their headers
  const uint32_t pc = p.pc;
  for (uint32_t r = lane; r < nu; r += kWave) {
    const uint32_t k = kind[r];
    const uint32_t base = r * a.img_dw * 32u;
    uint32_t lb = kBad, le = kBad, nb = nhead[r];
    if (k == 1u) {
      const uint32_t *hdr = stg + r * a.img_dw;
      uint32_t ones = 0;
      for (uint32_t d = 0; d < a.S / 32u; ++d) ones += __builtin_popcount(hdr[d]);
      if (a.S & 31u) ones += __builtin_popcount(hdr[a.S / 32u] & ((1u << (a.S & 31u)) - 1u));
      const uint32_t bits = a.S * (W + 1) - pc * ones;
      if (bits < a.row_bytes * 8u) {
        lb = base;
        le = base + bits;
        nb = (bits + 127u) / 128u;
      } else {
        err |= IBP_DEVERR_CORRUPT;  // a compressed slot can never be as long as the raw row
        kind[r] = 0u;
      }
    }
    lbeg[r] = lb;
    lend[r] = le;
    nblk[r] = nb;
  }
  wave_lds_sync();
  // second round: the rest of each compressed row
  for (uint32_t f0 = 0; f0 < total; f0 += 4 * kWave) {
    uint4 tmp[4];
    uint32_t dst[4];
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u) {
      const uint32_t f = f0 + u * kWave + lane;
      const uint32_t r = f / row_blocks, j = f - r * row_blocks;
      dst[u] = kBad;
      if (f < total && kind[r] == 1u && j >= nhead[r] && j < nblk[r]) {
        tmp[u] = load16(a.slots, slot0[r] + j);
        dst[u] = r * a.img_dw + 4u * j;
      }
    }
#pragma unroll
    for (uint32_t u = 0; u < 4; ++u)
      if (dst[u] != kBad) *reinterpret_cast<uint4 *>(stg + dst[u]) = tmp[u];
  }
  wave_lds_sync();
  // d. raw rows straight out, compressed rows decoded
  T *out = static_cast<T *>(a.out) + u0 * a.S;
  for (uint32_t r = 0; r < nu; ++r) {
    if (uniform(kind[r]) != 2u) continue;
    uint4 *o = reinterpret_cast<uint4 *>(out + (uint64_t)r * a.S);
    const uint4 *s = reinterpret_cast<const uint4 *>(stg + r * a.img_dw);
    for (uint32_t q = lane; q < row_blocks; q += kWave) store_nt16(o + q, s[q]);
  }
  DecodeArgs da{};
  da.S = a.S;
  da.s_log2 = a.s_log2;
  const uint32_t nch = nu * a.S;
  if constexpr (kMode == kModeLargeS)
    err |= decode_large_s<T, NR>(da, p, stg, lbeg, lend, nu, nch, out, lane);
  else if constexpr (kMode == kModeSmallS)
    err |= decode_small_s<T, true, NR>(da, p, stg, lbeg, lend, nch, out, lane);
  else
    err |= decode_general<T, true>(da, p, stg, lbeg, lend, gseg, nch, out, lane);
  if (err && a.err) atomicOr(a.err, err);
}

// ------------------------------------------------------------------ launch

struct Launch {
  dim3 grid;
  size_t shmem;
  hipStream_t s;
};

template <typename T, uint32_t NR>
hipError_t go_enc(const SlotArgs &a, const CodecParams &p, const Launch &l) {
  hipLaunchKernelGGL((encode_slots_kernel<T, NR>), l.grid, dim3(kBlock), l.shmem, l.s, a, p);
  return hipGetLastError();
}

template <typename T>
hipError_t go_enc_runs(const SlotArgs &a, const CodecParams &p, const Launch &l) {
  switch (runs_bucket(p.runs.n)) {
    case 1: return go_enc<T, 1>(a, p, l);
    case 2: return go_enc<T, 2>(a, p, l);
    case 3: return go_enc<T, 3>(a, p, l);
    case 4: return go_enc<T, 4>(a, p, l);
    case 5: return go_enc<T, 5>(a, p, l);
    case 6: return go_enc<T, 6>(a, p, l);
    case 7: return go_enc<T, 7>(a, p, l);
    case 8: return go_enc<T, 8>(a, p, l);
    default: return go_enc<T, 0>(a, p, l);
  }
}

template <typename T, uint32_t M, uint32_t NR>
hipError_t go_dec(const SlotArgs &a, const CodecParams &p, const Launch &l) {
  hipLaunchKernelGGL((decode_slots_kernel<T, M, NR>), l.grid, dim3(kBlock), l.shmem, l.s, a, p);
  return hipGetLastError();
}

template <typename T, uint32_t M>
hipError_t go_dec_runs(const SlotArgs &a, const CodecParams &p, const Launch &l) {
  switch (runs_bucket(p.runs.n)) {
    case 1: return go_dec<T, M, 1>(a, p, l);
    case 2: return go_dec<T, M, 2>(a, p, l);
    case 3: return go_dec<T, M, 3>(a, p, l);
    case 4: return go_dec<T, M, 4>(a, p, l);
    case 5: return go_dec<T, M, 5>(a, p, l);
    case 6: return go_dec<T, M, 6>(a, p, l);
    case 7: return go_dec<T, M, 7>(a, p, l);
    case 8: return go_dec<T, M, 8>(a, p, l);
    default: return go_dec<T, M, 0>(a, p, l);
  }
}

template <typename T>
hipError_t go_dec_mode(const SlotArgs &a, const CodecParams &p, const Launch &l) {
  if (a.S % kWave == 0) return go_dec_runs<T, kModeLargeS>(a, p, l);
  if (kWave % a.S == 0) return go_dec_runs<T, kModeSmallS>(a, p, l);
  return go_dec<T, kModeGeneral, 0>(a, p, l);
}

Launch make_launch(const SlotArgs &a, hipStream_t s, bool &ok) {
  const uint64_t tiles = (a.n_units + a.G - 1) / a.G;
  const uint64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  ok = blocks <= 0x7FFFFFFFull;
  return Launch{dim3((uint32_t)blocks), (size_t)a.wave_dw * 4 * kWavesPerBlock, s};
}

}  // namespace

hipError_t launch_encode_slots(const SlotArgs &a, const CodecParams &p, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  bool ok = false;
  const Launch l = make_launch(a, s, ok);
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = launch_zero(a.flags, (a.n_rows + 63) / 64, s);
  if (e != hipSuccess) return e;
  if (p.W == 16) return go_enc_runs<uint16_t>(a, p, l);
  return p.W == 32 ? go_enc_runs<uint32_t>(a, p, l) : go_enc_runs<uint64_t>(a, p, l);
}

hipError_t launch_decode_slots(const SlotArgs &a, const CodecParams &p, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  bool ok = false;
  const Launch l = make_launch(a, s, ok);
  if (!ok) return hipErrorInvalidValue;
  if (a.S % kWave != 0 && kWave % a.S == 0 && a.s_log2 == kNotPow2) return hipErrorInvalidValue;
  if (p.W == 16) return go_dec_mode<uint16_t>(a, p, l);
  return p.W == 32 ? go_dec_mode<uint32_t>(a, p, l) : go_dec_mode<uint64_t>(a, p, l);
}

}  // namespace ibp
