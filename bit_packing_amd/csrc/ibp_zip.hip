// ibp_zip.hip -- the comparison codec: exponent coding of BF16 tensors as on the
// page "ZipCCL: Efficient Lossless Data Compression of Communication Collectives
// for Accelerating LLM Training", section 2 (Metodologia), A and B, on one GPU
// and without collectives.
//
// A BF16 word splits into a sign-mantissa byte and its 8-bit exponent.  The 7
// exponents of a table derived from the tensor's standard deviation get 3-bit
// codes 1..7; any other exponent gets code 0 and is stored whole, in element
// order, in an escape array.  Per block of 4096 elements the codes are kept as
// three bit planes of 4096 bits; eoff[j] counts the escapes before block j.
//
// A 256-thread workgroup decodes one block, and compresses kZipWG consecutive
// blocks; in every block thread t handles the two groups of 8 consecutive
// elements [q*2048 + 8t, +8), q = 0, 1, so sign-mantissa bytes, plane bytes and
// BF16 words move as 8-, 1- and 16-byte accesses.  The escapes of a thread are
// ranked by a block scan of two 16-bit counts packed in one word (group 0 low,
// group 1 high), and the first escape of the compressor's workgroup by a
// decoupled look-back over the workgroups (the decompressor reads eoff).
#include "ibp_device.h"

namespace ibp {
namespace {

using namespace dev;

constexpr uint32_t kGroup = 8;                          // consecutive elements per thread and group
constexpr uint32_t kHalf = kZipBlock / 2;               // elements per group pass
constexpr uint32_t kPlane = kZipBlock / 8;              // bytes per code plane

// Inclusive scan of v over the workgroup (256 threads); *total gets the sum.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t lane, uint32_t wave, uint32_t *wsum,
                                               uint32_t *total) {
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  uint32_t pre = 0, all = 0;
#pragma unroll
  for (uint32_t w = 0; w < kWavesPerBlock; ++w) {
    const uint32_t s = wsum[w];
    if (w < wave) pre += s;
    all += s;
  }
  *total = all;
  return pre + x;
}

__global__ void __launch_bounds__(kBlock) zip_encode_kernel(ZipArgs a) {
  // exponent -> code c as plane bits (c & 1, c >> 1 & 1, c >> 2 & 1 at bits 0, 8,
  // 16), or bit 24 for an exponent outside the table (an escape): OR-ing
  // lut[e_k] << k over the 8 elements of a group leaves the group's three plane
  // bytes in bytes 0..2 and its escape mask in byte 3
  __shared__ uint32_t lut[256];
  __shared__ uint32_t wsum[kZipWG][kWavesPerBlock];
  __shared__ uint64_t s_excl;
  __shared__ uint32_t s_failed;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = uniform(tid / kWave);
  lut[tid] = 1u << 24;
  __syncthreads();
  if (tid < 7) {
    const uint32_t c = tid + 1;
    lut[a.table[tid]] = (c & 1u) | ((c >> 1) & 1u) << 8 | ((c >> 2) & 1u) << 16;
  }
  __syncthreads();
  // workgroup g compresses blocks [j0, j0 + nbw); grid == workgroups, the
  // look-back over workgroups relies on their order
  const uint64_t g = blockIdx.x;
  const uint64_t j0 = g * kZipWG;
  const uint32_t nbw = (uint32_t)min((uint64_t)kZipWG, a.nblk - j0);

  // 1. every block's BF16 words first
  uint32_t ws[kZipWG][2][4];
#pragma unroll
  for (uint32_t b = 0; b < kZipWG; ++b) {
    const uint64_t e0 = (j0 + b) * kZipBlock;
    const uint32_t nb = b < nbw ? (uint32_t)min((uint64_t)kZipBlock, a.n - e0) : 0u;
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
      const uint32_t t0 = q * kHalf + kGroup * tid;
      if (t0 + kGroup <= nb) {
        const uint4 w = *reinterpret_cast<const uint4 *>(a.in + e0 + t0);
        ws[b][q][0] = w.x;
        ws[b][q][1] = w.y;
        ws[b][q][2] = w.z;
        ws[b][q][3] = w.w;
      } else {
#pragma unroll
        for (uint32_t k = 0; k < kGroup / 2; ++k) {
          const uint32_t lo = t0 + 2 * k < nb ? a.in[e0 + t0 + 2 * k] : 0u;
          const uint32_t hi = t0 + 2 * k + 1 < nb ? a.in[e0 + t0 + 2 * k + 1] : 0u;
          ws[b][q][k] = lo | (hi << 16);
        }
      }
    }
  }
  // 2. per block: sign-mantissa and exponent bytes, codes, escape ranks (a block
  //    scan of the two groups' counts packed in one word, group 0 low)
  uint32_t smw[kZipWG][2][2], ex[kZipWG][2][2], acc[kZipWG][2];
  uint32_t escm[kZipWG];       // bit q*8 + k: element k of group q is an escape
  uint32_t rank[kZipWG][2];    // escapes of the workgroup before this thread's group q
  uint32_t btot[kZipWG];       // escapes per block
  uint32_t wtot = 0;           // escapes of the workgroup
#pragma unroll
  for (uint32_t b = 0; b < kZipWG; ++b) {
    const uint32_t nb = b < nbw ? (uint32_t)min((uint64_t)kZipBlock, a.n - (j0 + b) * kZipBlock) : 0u;
    uint32_t packed = 0;
    escm[b] = 0;
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
      const uint32_t t0 = q * kHalf + kGroup * tid;
      // two elements per word: sign-mantissa byte (sign at bit 7) and exponent in
      // the low byte of each 16-bit half, then four of them gathered into one word
      uint32_t sp[4], ep[4];
#pragma unroll
      for (uint32_t k = 0; k < 4; ++k) {
        sp[k] = (ws[b][q][k] & 0x007F007Fu) | ((ws[b][q][k] >> 8) & 0x00800080u);
        ep[k] = (ws[b][q][k] >> 7) & 0x00FF00FFu;
      }
      smw[b][q][0] = __builtin_amdgcn_perm(sp[1], sp[0], 0x06040200u);
      smw[b][q][1] = __builtin_amdgcn_perm(sp[3], sp[2], 0x06040200u);
      ex[b][q][0] = __builtin_amdgcn_perm(ep[1], ep[0], 0x06040200u);
      ex[b][q][1] = __builtin_amdgcn_perm(ep[3], ep[2], 0x06040200u);
      uint32_t c = 0;
#pragma unroll
      for (uint32_t k = 0; k < kGroup; ++k) c |= lut[(ex[b][q][k / 4] >> (8 * (k % 4))) & 0xFFu] << k;
      const uint32_t valid = nb > t0 ? min(nb - t0, kGroup) : 0u;  // elements of the group inside the block
      const uint32_t em = (c >> 24) & ((1u << valid) - 1u);
      acc[b][q] = c & (((1u << valid) - 1u) * 0x010101u);  // elements past nb have code 0
      escm[b] |= em << (q * kGroup);
      packed += (uint32_t)__builtin_popcount(em) << (16 * q);
    }
    uint32_t total = 0;
    const uint32_t incl = block_scan(packed, lane, wave, wsum[b], &total);
    const uint32_t excl_t = incl - packed;
    const uint32_t tot0 = total & 0xFFFFu;
    rank[b][0] = wtot + (excl_t & 0xFFFFu);
    rank[b][1] = wtot + tot0 + (excl_t >> 16);
    btot[b] = tot0 + (total >> 16);
    wtot += btot[b];
  }
  // the workgroup's escape count first, published at once for the successors'
  // look-back; then the sign-mantissa bytes and code planes, which need no offset
  if (tid == 0) lookback_publish(a.status, a.st_lg, g, wtot);
#pragma unroll
  for (uint32_t b = 0; b < kZipWG; ++b) {
    if (b >= nbw) continue;
    const uint64_t j = j0 + b, e0 = j * kZipBlock;
    const uint32_t nb = (uint32_t)min((uint64_t)kZipBlock, a.n - e0);
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
      const uint32_t t0 = q * kHalf + kGroup * tid;
      uint8_t *smo = a.sm + e0 + t0;
      if (t0 + kGroup <= nb) {
        store_nt8(smo, make_uint2(smw[b][q][0], smw[b][q][1]));
      } else {
        for (uint32_t k = 0; t0 + k < nb; ++k) smo[k] = (uint8_t)(smw[b][q][k / 4] >> (8 * (k % 4)));
      }
      uint8_t *cp = a.codes + j * (3 * kPlane) + q * (kHalf / 8) + tid;
      cp[0] = (uint8_t)acc[b][q];
      cp[kPlane] = (uint8_t)(acc[b][q] >> 8);
      cp[2 * kPlane] = (uint8_t)(acc[b][q] >> 16);
    }
  }
  if (wave == 0) {
    bool timed_out = false;
    const uint64_t excl = g == 0 ? 0ull
                                 : lookback_finish(a.status, a.st_lg, a.control, a.err, g, (int64_t)g - 1, 0, wtot,
                                                   a.wait_limit, lane, timed_out);
    if (lane == 0) {
      s_excl = excl;
      s_failed = timed_out ? 1u : 0u;
    }
  }
  __syncthreads();
  if (s_failed != 0u) {
    // no valid escape offset: no escapes are stored, and the blocks' offsets become
    // ~0, which the decoder refuses
    if (tid == 0) {
      for (uint32_t b = 0; b < nbw; ++b) a.eoff[j0 + b] = ~0ull;
      if (j0 + nbw == a.nblk) a.eoff[a.nblk] = ~0ull;
    }
    return;
  }
  const uint64_t base = s_excl;
  if (tid == 0) {
    uint64_t o = base;
    for (uint32_t b = 0; b < nbw; ++b) {
      a.eoff[j0 + b] = o;
      o += btot[b];
    }
    if (j0 + nbw == a.nblk) a.eoff[a.nblk] = o;
  }
#pragma unroll
  for (uint32_t b = 0; b < kZipWG; ++b) {
#pragma unroll
    for (uint32_t q = 0; q < 2; ++q) {
      uint64_t r = base + rank[b][q];
      for (uint32_t m = (escm[b] >> (q * kGroup)) & 0xFFu; m; m &= m - 1u) {
        const uint32_t k = (uint32_t)__builtin_ctz(m);
        a.esc[r++] = (uint8_t)(ex[b][q][k / 4] >> (8 * (k % 4)));
      }
    }
  }
}

// Bits 0..3 of x spread to bit 0 of bytes 0..3 (bit k -> bit 8k): the shifted
// copies x, x << 7, x << 14, x << 21 do not overlap, so the product has no carries.
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return __umul24(x & 0xFu, 0x00204081u) & 0x01010101u; }

// Bytes i of the result: 0 if byte i of x is 0, else 0x80 (bytes of x at most 0x7F).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) { return (x + 0x7F7F7F7Fu) & 0x80808080u; }

// BF16 words of two elements from their sign-mantissa and exponent bytes placed
// in the low bytes of the 16-bit halves of sp and ep.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t sp, uint32_t ep) {
  return ((sp << 8) & 0x80008000u) | (ep << 7) | (sp & 0x007F007Fu);
}

__global__ void __launch_bounds__(kBlock) zip_decode_kernel(ZipArgs a) {
  __shared__ uint32_t wsum[kWavesPerBlock];
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = uniform(tid / kWave);
  // exponent of code c in byte c of (thi:tlo); byte 0 (escape) is 0
  const uint32_t tlo = ((uint32_t)a.table[0] << 8) | ((uint32_t)a.table[1] << 16) | ((uint32_t)a.table[2] << 24);
  const uint32_t thi = (uint32_t)a.table[3] | ((uint32_t)a.table[4] << 8) | ((uint32_t)a.table[5] << 16) |
                       ((uint32_t)a.table[6] << 24);
  const uint64_t j = blockIdx.x;
  const uint64_t e0 = j * kZipBlock;
  const uint32_t nb = (uint32_t)min((uint64_t)kZipBlock, a.n - e0);
  // every load that does not depend on the escape ranks is issued first
  const uint64_t E0 = a.eoff[j], E1 = a.eoff[j + 1];
  uint32_t pb[2][3];
  uint32_t sm[2][2];
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    const uint8_t *cp = a.codes + j * (3 * kPlane) + q * (kHalf / 8) + tid;
    pb[q][0] = cp[0];
    pb[q][1] = cp[kPlane];
    pb[q][2] = cp[2 * kPlane];
    sm[q][0] = sm[q][1] = 0;
    if (t0 + kGroup <= nb) {
      const uint2 w = *reinterpret_cast<const uint2 *>(a.sm + e0 + t0);
      sm[q][0] = w.x;
      sm[q][1] = w.y;
    } else {
      for (uint32_t k = 0; t0 + k < nb; ++k) sm[q][k / 4] |= (uint32_t)a.sm[e0 + t0 + k] << (8 * (k % 4));
    }
  }
  // codes of elements 4h..4h+3 of group q as the bytes of cb[q][h], and the escapes
  // (code 0 of an element inside the block) as 0x80 bytes of esc[q][h]
  uint32_t cb[2][2], esc[2][2];
  uint32_t packed = 0;
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    const uint32_t valid = nb > t0 ? min(nb - t0, kGroup) : 0u;  // elements of the group inside the block
    uint32_t n = 0;
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      cb[q][h] = spread4(pb[q][0] >> (4 * h)) | (spread4(pb[q][1] >> (4 * h)) << 1) |
                 (spread4(pb[q][2] >> (4 * h)) << 2);
      const uint32_t vh = valid > 4 * h ? min(valid - 4 * h, 4u) : 0u;  // valid elements of this word
      const uint32_t in_block = vh >= 4 ? 0xFFFFFFFFu : ((1u << (8 * vh)) - 1u);
      esc[q][h] = ~nonzero_bytes(cb[q][h]) & 0x80808080u & in_block;
      n += __builtin_popcount(esc[q][h]);
    }
    packed += n << (16 * q);
  }
  uint32_t total;
  const uint32_t incl = block_scan(packed, lane, wave, wsum, &total);
  const uint32_t excl_t = incl - packed;
  const uint32_t tot0 = total & 0xFFFFu, agg = tot0 + (total >> 16);
  if (E1 < E0 || E1 - E0 != agg || E1 > a.esc_bytes) {
    if (tid == 0 && a.err) atomicOr(a.err, IBP_DEVERR_CORRUPT);
    return;  // block not decoded
  }
#pragma unroll
  for (uint32_t q = 0; q < 2; ++q) {
    const uint32_t t0 = q * kHalf + kGroup * tid;
    if (t0 >= nb) continue;
    // exponents: table bytes by code, then this thread's escapes (consecutive in the
    // escape array per group) in element order
    uint32_t ex[2];
    uint64_t r = E0 + (q == 0 ? (excl_t & 0xFFFFu) : tot0 + (excl_t >> 16));
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      ex[h] = __builtin_amdgcn_perm(thi, tlo, cb[q][h]);
      for (uint32_t m = esc[q][h]; m; m &= m - 1u) {
        const uint32_t sh = (uint32_t)__builtin_ctz(m) - 7u;  // 8 * (byte index)
        ex[h] |= (uint32_t)a.esc[r++] << sh;
      }
    }
    // pairs of elements: sign-mantissa and exponent bytes moved to the 16-bit halves
    const uint32_t w0 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][0], 0x0C010C00u), __builtin_amdgcn_perm(0u, ex[0], 0x0C010C00u));
    const uint32_t w1 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][0], 0x0C030C02u), __builtin_amdgcn_perm(0u, ex[0], 0x0C030C02u));
    const uint32_t w2 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][1], 0x0C010C00u), __builtin_amdgcn_perm(0u, ex[1], 0x0C010C00u));
    const uint32_t w3 = bf16_pair(__builtin_amdgcn_perm(0u, sm[q][1], 0x0C030C02u), __builtin_amdgcn_perm(0u, ex[1], 0x0C030C02u));
    uint16_t *o = a.out + e0 + t0;
    if (t0 + kGroup <= nb) {
      store_nt16(o, make_uint4(w0, w1, w2, w3));
    } else {
      const uint32_t w[4] = {w0, w1, w2, w3};
      for (uint32_t k = 0; t0 + k < nb; ++k) o[k] = (uint16_t)(w[k / 2] >> (16 * (k % 2)));
    }
  }
}

}  // namespace

hipError_t launch_zip_encode(const ZipArgs &a, hipStream_t s) {
  if (a.nblk == 0) return hipSuccess;
  if (a.nblk > 0x7FFFFFFFull) return hipErrorInvalidValue;
  // clear the control words and status words (a kernel, not a memset node)
  const uint64_t groups = (a.nblk + kZipWG - 1) / kZipWG;
  hipError_t e = launch_zero(reinterpret_cast<uint64_t *>(a.control), 1 + status_words(groups), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zip_encode_kernel, dim3((uint32_t)groups), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zip_decode(const ZipArgs &a, hipStream_t s) {
  if (a.nblk == 0) return hipSuccess;
  if (a.nblk > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zip_decode_kernel, dim3((uint32_t)a.nblk), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace ibp
