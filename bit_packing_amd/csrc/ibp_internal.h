// ibp_internal.h -- definitions shared by the host launch code and the gfx950
// kernels of the IBP codec.  Not part of the public ABI (that is include/ibp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ibp {

constexpr uint32_t kWave = 64;          // CDNA4 wavefront width
constexpr uint32_t kBlock = 256;        // threads per workgroup for every kernel
constexpr uint32_t kWavesPerBlock = kBlock / kWave;
constexpr uint32_t kMaxRuns = 32;       // at most 32 runs of free bits in a 64-bit chunk

// Compression: a workgroup of enc_threads() threads sizes, offsets and packs a
// tile of 16 chunks per thread.  Measured on the workloads: 512 threads beat 256
// by 3-10% with one Mask; with position-dependent metadata, whose tables and
// per-chunk prefixes also live in LDS, 256 is fastest at W = 32 and 64 (512: 17-50%
// slower) and 512 at W = 16 (4.4 -> 3.3 ms per 2^30 chunks); 128 and 64 threads were
// 10-50% slower, their per-tile costs spread over fewer chunks.  The W = 16 pair
// form (two chunks per lane) takes 32 chunks per thread, so a tile still moves
// 32 KB of input.
constexpr uint32_t enc_threads(bool pos, uint32_t W, bool big = false) {
  return big ? 1024u : (pos && W != 16 ? 256u : 512u);
}
constexpr uint32_t enc_tile_chunks(bool pos, bool pair, uint32_t W, uint32_t halves = 1, bool big = false) {
  return (pair || (halves == 2 && W == 32) ? 32u : 16u) * enc_threads(pos, W, big);
}
// From 2^23 chunks on (ibp_set_halves_min_chunks; smaller launches do not fill the
// GPU and finish sooner with one-image tiles), a compression tile of 32- or 64-bit
// chunks with one Mask and S a power of two is packed and stored in two halves
// (segments end at the middle) through an LDS image of half the size.  64-bit chunks: 8192-chunk tiles, whose full-size image
// (8192 chunks x 65 bits) would leave room for two workgroups per CU, the half-size
// one for four.  32-bit chunks: 16384-chunk tiles (32 per thread) through the
// image of 8192, so a tile moves 64 KB of input, as at W = 64, with half the
// look-backs per byte of 8192-chunk tiles.  A tile whose stream fits the half-size
// image is packed whole before its look-back and stored once.  Position metadata
// takes the same form at W = 64 (same tile, half the image: the registers, not the
// LDS, then bound the workgroups per CU; ids 2.00 -> 1.79 ms, llm 1.38 -> 1.29 ms,
// S = 32 feature rows 0.345 -> 0.305 ms); at W = 32 its two-half kernels need 139+
// VGPRs, while the one-image ones already fit six waves per SIMD.
inline uint32_t enc_halves(bool pos, bool pair, uint32_t W, uint32_t S) {
  return (W == 64 || (W == 32 && !pos)) && !pair && S != 0 && (S & (S - 1)) == 0 ? 2u : 1u;
}
// A tile saves at most popcount(Mask) bits per chunk, so only when popcount(Mask) >
// (W + 1) / 2 can a whole tile fit the half-size image.  For such 64-bit chunks the
// tile doubles (1024 threads, 16384 chunks, two workgroups per CU): each look-back
// then covers 128 KB (measured on the id stream, which fits: 1.19 -> 1.12 ms; tiles
// that do not fit ran 2-13% slower at this size, so the others keep 512 threads).
inline bool enc_big(uint32_t W, uint32_t halves, uint32_t pc) { return halves == 2 && W == 64 && 2 * pc > W + 1; }
// Decompression tile: a wavefront decodes about this many chunks at a time,
// with at most this many segments (rows) per tile.
constexpr uint32_t kDecTileChunks = 512;
constexpr uint32_t kDecMaxUnits = 128;
constexpr uint32_t kGatherMaxRows = 8;   // rows per wavefront of a gather from HBM
// Metadata count kernel: at most this many workgroups (one per CU) write partial counts.
constexpr uint32_t kMetaMaxBlocks = 256;
constexpr uint32_t kMetaThreads = 1024;  // threads per workgroup of the one-count kernel

// Look-back status words, one per tile, are spread so that tiles in flight together
// do not share a 128-byte line: tile t's word is word t / 2^lg of line t mod 2^lg
// (2^lg lines of 16 words, 2^lg >= ntiles / 16), so the 16 tiles of a line lie 2^lg
// apart.  Packed 16 to a line, consecutive tiles' publishing stores and their
// successors' polling loads contended for the same lines (measured: compression
// 8-10% slower on every workload).
inline uint32_t status_lg(uint64_t ntiles) {
  uint32_t lg = 0;
  while ((16ull << lg) < ntiles) ++lg;
  return lg;
}
inline uint64_t status_words(uint64_t ntiles) { return 16ull << status_lg(ntiles); }  // < 2 ntiles + 32
// Status words of the compression look-back: 2-bit flag above a 62-bit value.
constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagPrefix = 2ull << 62;
constexpr uint64_t kValueMask = (1ull << 62) - 1;
// Hand-over word of the boundary between tiles t and t + 1 (when it falls inside a
// dword): each tile ORs in its bits of that dword (low 32 bits) and its flag.
constexpr uint64_t kTailReady = 1ull << 63;  // tile t's bits are in
constexpr uint64_t kHeadReady = 1ull << 62;  // tile t + 1's bits are in

// The free (non-Mask) positions of a chunk split into maximal runs of
// consecutive bits.  Run r sits at chunk bits [pos_r, pos_r + len_r) and at
// payload bits [cum_r, cum_r + len_r), cum_r = total length of the runs below it.
// Stored as the payload-side mask lowbits(len_r) << cum_r and the shift
// pos_r - cum_r (never negative), so extract and deposit are one shift, one AND
// and one OR per run.
struct Runs {
  uint64_t pmask[kMaxRuns];
  uint32_t shift[kMaxRuns];
  uint32_t n;
};

struct CodecParams {
  uint64_t mask;
  uint64_t bitval;
  uint32_t W;   // 16, 32 or 64
  uint32_t pc;  // popcount(mask)
  Runs runs;
};

struct MetaArgs {
  const void *in;
  uint64_t n;          // sample chunks
  uint64_t *partial;   // [blocks][W] partial counts
  uint64_t *result;    // [64 counts][mask][bitval]
  uint64_t k;          // majority count needed for an invariant bit
  uint32_t W;
  uint32_t blocks;
};

struct EncodeArgs {
  const void *in;
  uint32_t *stream;    // dword view of the output stream
  uint64_t *off;       // nseg + 1 bit offsets
  uint64_t *status;    // status_words(ntiles) look-back words, tile t's at status_slot(t, st_lg)
  uint64_t *tails;     // ntiles hand-over words (the dword shared by tiles t and t + 1)
  uint32_t *control;   // [0] unused, [1] abort flag
  uint32_t *err;       // optional
  const uint64_t *pmask;    // position-dependent metadata: Mask_i, i < S (device), else null
  const uint64_t *pbitval;  // Bitval_i, i < S
  uint64_t n_chunks;
  uint64_t nseg;
  uint64_t ntiles;
  uint32_t S;
  uint32_t s_log2;     // log2(S) when S is a power of two, else kNotPow2
  uint32_t G;          // segments per tile
  uint32_t tile_chunks;
  uint32_t obuf_dw;    // LDS dwords for the packed tile
  uint32_t pair;       // 1: W = 16 chunk pairs (one Mask, S a multiple of 64, input 4-byte aligned)
  uint32_t wait_limit; // look-back polls of one unpublished predecessor before a tile gives up
  uint32_t st_lg;      // status_lg(ntiles)
  uint32_t halves;     // 2: the tile is packed and stored in two halves through a half-size image
  uint32_t big;        // 1: 1024-thread tiles (enc_big)
};

struct DecodeArgs {
  const uint64_t *pmask;    // position-dependent metadata: Mask_i, i < S (device), else null
  const uint64_t *pbitval;  // Bitval_i, i < S
  const uint8_t *stream;
  uint64_t stream_bytes;
  const uint64_t *off;
  const int64_t *ids;  // gather: segment id of each output row
  void *out;
  uint32_t *err;       // optional
  uint64_t n_chunks;   // chunks written in total
  uint64_t n_units;    // contiguous: segments; gather: rows
  uint64_t nseg;       // segments in the stream
  uint32_t S;
  uint32_t s_log2;
  uint32_t G;          // units per wave tile
  uint32_t stage_dw;   // LDS staging dwords per wave
  uint32_t slot_dw;    // gather: staging dwords per row
  uint32_t sb_magic;   // gather: ceil(2^32 / (slot_dw / 4)), for a division by the slot's block count
  uint32_t wave_dw;    // LDS dwords per wave in total
};

struct RawGatherArgs {
  const uint8_t *src;
  const int64_t *ids;
  uint8_t *out;
  uint32_t *err;
  uint64_t row_blocks; // row size in 16-byte blocks
  uint64_t n_rows;
  uint64_t n_ids;
};

// Fixed-slot layout: row r of the table owns row_bytes bytes at slots + r * row_bytes.
struct SlotArgs {
  const void *in;      // compress: the raw rows
  uint8_t *slots;      // compress: written; decompress: read (device or pinned host memory)
  uint64_t *flags;     // 1 bit per row in 64-bit words (device memory)
  const int64_t *ids;  // decompress: row ids
  void *out;           // decompress: output rows
  uint32_t *err;       // optional
  uint64_t n_rows;     // rows in the table
  uint64_t n_units;    // compress: n_rows; decompress: n_ids
  uint32_t S;
  uint32_t s_log2;
  uint32_t G;          // rows per wavefront tile
  uint32_t row_bytes;  // S * W / 8, a multiple of 16
  uint32_t img_dw;     // LDS dwords per row
  uint32_t wave_dw;    // LDS dwords per wavefront
  uint32_t head_blocks;  // decompress: 16-byte blocks read before the header is known
};

// Comparison codec (BF16 exponent coding): elements per block.
constexpr uint32_t kZipBlock = 4096;
constexpr uint32_t kZipWG = 4;  // blocks per compressor workgroup (one look-back each)

struct ZipArgs {
  const uint16_t *in;  // compress: BF16 words (16-byte aligned)
  uint16_t *out;       // decompress: BF16 words (16-byte aligned)
  uint8_t *sm;         // sign-mantissa bytes, n (8-byte aligned)
  uint8_t *codes;      // three 512-byte code planes per block
  uint8_t *esc;        // escape exponents
  uint64_t esc_bytes;  // decompress: readable escape bytes
  uint64_t *eoff;      // nblk + 1 escape offsets
  uint64_t *status;    // compress: status_words(workgroups) look-back words (status_slot, st_lg)
  uint32_t *control;   // compress: [0] unused, [1] abort flag
  uint32_t *err;       // optional
  uint64_t n;
  uint64_t nblk;
  uint32_t table[7];   // exponents of codes 1..7, distinct
  uint32_t wait_limit; // compress: look-back polls of one unpublished predecessor before giving up
  uint32_t st_lg;      // compress: status_lg(workgroups)
};

constexpr uint32_t kNotPow2 = 0xFFFFFFFFu;

// Launchers (ibp_meta.hip, ibp_encode.hip, ibp_decode.hip, ibp_decode_pos.hip,
// ibp_slots.hip, ibp_zip.hip).  Each returns the hipError_t of its launch(es).
hipError_t launch_meta(const MetaArgs &a, hipStream_t s);
hipError_t launch_meta_pos(const MetaArgs &a, uint32_t S, uint64_t *d_mask, uint64_t *d_bitval, hipStream_t s);
hipError_t launch_encode(const EncodeArgs &a, const CodecParams &p, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, const CodecParams &p, bool gather, hipStream_t s);
hipError_t launch_decode_pos(const DecodeArgs &a, const CodecParams &p, hipStream_t s);  // ibp_decode_pos.hip
hipError_t launch_raw_gather(const RawGatherArgs &a, hipStream_t s);
hipError_t launch_zero(uint64_t *p, uint64_t n, hipStream_t s);
hipError_t launch_zip_encode(const ZipArgs &a, hipStream_t s);  // ibp_zip.hip
hipError_t launch_zip_decode(const ZipArgs &a, hipStream_t s);
hipError_t launch_encode_slots(const SlotArgs &a, const CodecParams &p, hipStream_t s);  // ibp_slots.hip
hipError_t launch_decode_slots(const SlotArgs &a, const CodecParams &p, hipStream_t s);

}  // namespace ibp
