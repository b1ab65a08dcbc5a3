/*
 * ibp.h -- C ABI of the MI355X (gfx950) Invariant Bit Packing (IBP) codec.
 *
 * The method is the one summarised in "Riduzione del Collo di Bottiglia della
 * Memoria GPU con la Compressione Lossless per il ML" (gist.science, paper
 * 2605.30728), section "Algoritmo Core":
 *   1. Preprocessing: find the bit positions of a W-bit chunk that keep one value
 *      over at least a fraction T of a sample batch -> Mask, and their values ->
 *      Bitval (ibp_build_metadata);
 *   2. Compression: a chunk whose Mask bits equal Bitval loses those bits; every
 *      chunk carries a participation bit (ibp_compress);
 *   3. Decompression: a wavefront stages a contiguous compressed segment in LDS,
 *      finds each lane's bit offset with a wave-wide prefix count and re-inserts
 *      the Bitval bits (ibp_decompress; ibp_decompress_gather for rows read
 *      straight from pinned host memory, the "PCIe Transfer Compression" mode of
 *      section "Integrazione del Sistema").
 *
 * Compressed format (shared with nothing else; every call below produces or
 * consumes exactly this):
 *   - chunk i is the little-endian word at bytes [i*W/8, (i+1)*W/8) of the input;
 *   - chunks are grouped into segments of S consecutive chunks (the last segment
 *     may be shorter);
 *   - a segment of m chunks is: m participation bits (1 = compressed), in chunk
 *     order, then the m payloads back to back in chunk order; a compressed
 *     chunk's payload is its W - popcount(Mask) non-Mask bits in increasing
 *     position order, a raw chunk's payload is all W bits;
 *   - stream bit q is bit (q % 8) of byte q / 8; fields are written low bit first;
 *   - segments are bit-contiguous (no padding); segment k starts at bit
 *     offsets[k]; offsets[nseg] is the total bit count; bits of the last byte
 *     above the total are 0.
 *   So the total is the sum over chunks of 1 + (compressed ? W - popcount(Mask) : W).
 *
 * Conventions for every call:
 *   - "d_" pointers are device memory (hipMalloc / torch CUDA tensors).  Stream
 *     inputs of the decoders may instead point to pinned host memory allocated
 *     with hipHostMalloc (read zero-copy over PCIe by the kernel).
 *   - hip_stream is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns, except ibp_build_metadata, which waits for
 *     its stream.
 *   - The caller allocates and frees every buffer; the library allocates no
 *     memory.  Workspaces are caller-provided, sized by the *_workspace_bytes
 *     queries; their contents on entry do not matter.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns an error code and enqueues nothing.  Calls never throw.
 *   - d_err_word (optional, may be NULL): a device uint32 that kernels OR error
 *     bits into (IBP_DEVERR_*).  The library never clears it.
 *   - All calls are stateless and may run concurrently on different streams.
 */
#ifndef IBP_H
#define IBP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define IBP_API __attribute__((visibility("default")))
#else
#define IBP_API
#endif

typedef enum {
  IBP_OK = 0,
  IBP_ERR_INVALID_ARG = 1, /* NULL pointer; W not 16, 32 or 64; S == 0 or S > IBP_MAX_S;
                              T not in (0.5, 1]; misaligned pointer; Bitval outside Mask */
  IBP_ERR_SIZE = 2,        /* byte count not a whole number of chunks; too many chunks */
  IBP_ERR_CAPACITY = 3,    /* stream capacity or workspace below the required size */
  IBP_ERR_DEVICE = 4       /* a HIP runtime call failed (kernel launch, copy, sync) */
} ibp_status_t;

/* Bits OR-ed into *d_err_word by the kernels. */
#define IBP_DEVERR_CORRUPT 1u   /* a segment's decoded length differs from its offset span,
                                   or its offsets are not monotone / exceed the stream */
#define IBP_DEVERR_BAD_ID 2u    /* a gather id is negative or >= n_segments; its row is skipped */
#define IBP_DEVERR_TIMEOUT 4u   /* compression: a tile gave up waiting for a predecessor's offset;
                                   its stream bits are not written and its offsets are set to
                                   ~0, which every decoder refuses (IBP_DEVERR_CORRUPT) */

/* Largest segment length (chunks per segment). */
#define IBP_MAX_S 1024u

/* Invariant-bit metadata of one dataset ("Algoritmo Core", step 1).  Only the low
 * W bits of mask and bitval are used; bitval must be 0 outside mask. */
typedef struct {
  uint32_t W;        /* chunk width in bits: 16, 32 or 64 */
  uint32_t reserved; /* must be 0 */
  uint64_t mask;     /* 1 = invariant position */
  uint64_t bitval;   /* value of each invariant position, 0 elsewhere */
} ibp_meta_t;

/* Human-readable name of a status code (static string). */
IBP_API const char *ibp_status_str(int status);

/* For tests of the compressors' give-up path only.  A compressing tile waits for
 * its predecessors' offsets (decoupled look-back); it gives up after `polls` polls
 * of one unpublished predecessor (default 2^20; 0xFFFFFFFF restores the default)
 * and reports IBP_DEVERR_TIMEOUT.  0 makes every tile that would wait give up at
 * once, so the give-up path runs without any kernel waiting.  Applies to calls
 * made after it, process-wide; returns the former value. */
IBP_API uint32_t ibp_set_wait_limit(uint32_t polls);

/* Compression tile form, for tuning and for tests that run both forms on small
 * inputs (the stream and offsets do not depend on it).  With one Mask, W = 32 or 64
 * and S a power of two, inputs of at least `n_chunks` chunks (default 2^23) take
 * the larger tiles packed in two halves, and smaller ones one-image tiles of 8192
 * chunks: a launch too small to fill the GPU is latency-bound and gains from more,
 * shorter tiles (measured: 65,536 chunks 9.5 us against 15.4 us; 2^26 chunks
 * 120 us against 150 us the other way; the cross-over lies between 2^22 and 2^23).
 * 0xFFFFFFFFFFFFFFFF restores the default.  Applies to calls made after it,
 * process-wide; returns the former value. */
IBP_API uint64_t ibp_set_halves_min_chunks(uint64_t n_chunks);

/* ceil(n_chunks / S); 0 when S == 0. */
IBP_API uint64_t ibp_num_segments(uint64_t n_chunks, uint32_t S);

/* Capacity a compressed stream of n_chunks W-bit chunks may need: the worst case
 * (every chunk raw, n*(W+1) bits) in bytes, rounded up to 16.  ibp_compress
 * requires stream_capacity >= this. */
IBP_API uint64_t ibp_max_stream_bytes(uint64_t n_chunks, uint32_t W);

/* Bytes of a stream of total_bits bits that the decoders may read:
 * ceil(total_bits / 8) rounded up to 16.  Pass at least the true length of the
 * buffer as stream_bytes; the kernels read nothing beyond stream_bytes. */
IBP_API uint64_t ibp_stream_bytes(uint64_t total_bits);

/* Workspace for ibp_build_metadata and ibp_compress. */
IBP_API uint64_t ibp_metadata_workspace_bytes(uint64_t n_sample_chunks, uint32_t W);
IBP_API uint64_t ibp_compress_workspace_bytes(uint64_t n_chunks, uint32_t S);

/*
 * Step 1 -- metadata ("Algoritmo Core", Preprocessing).
 *   d_samples: n_sample_chunks contiguous W-bit chunks (device, aligned to W/8).
 *   Position b is invariant when its majority value occurs in at least
 *   k = ceil(round(T * 10^6) * n / 10^6) samples; 0.5 < T <= 1.
 *   meta_out (host): W, mask, bitval.  counts_out (host, optional): W uint64, the
 *   number of samples with bit b set.
 *   Waits for hip_stream (the result is copied back to the host).
 */
IBP_API int ibp_build_metadata(const void *d_samples, uint64_t n_sample_chunks, uint32_t W, double T,
                               ibp_meta_t *meta_out, uint64_t *counts_out, void *d_workspace,
                               uint64_t workspace_bytes, void *hip_stream);

/*
 * Step 2 -- compression ("Algoritmo Core", Compressione).  One fused pass: each
 * tile of segments sizes itself, takes its bit offset from its predecessors by a
 * decoupled look-back, and packs.
 *   meta (host): as returned by ibp_build_metadata (or any valid Mask/Bitval).
 *   d_in: n_bytes of input (device, aligned to W/8); n_bytes % (W/8) == 0.
 *   S: chunks per segment, 1..IBP_MAX_S.
 *   d_stream: output, stream_capacity >= ibp_max_stream_bytes(n, W) bytes,
 *     aligned to 16.  Bytes past ceil(total/8) rounded up to 4 are not written.
 *   d_offsets: output, nseg + 1 uint64 bit offsets (device).
 *   d_workspace: ibp_compress_workspace_bytes(n, S) bytes (device).
 *   The total size is d_offsets[nseg] bits; copy it back when needed.
 */
IBP_API int ibp_compress(const ibp_meta_t *meta, const void *d_in, uint64_t n_bytes, uint32_t S,
                         void *d_stream, uint64_t stream_capacity, uint64_t *d_offsets,
                         void *d_workspace, uint64_t workspace_bytes, uint32_t *d_err_word,
                         void *hip_stream);

/*
 * Step 2 for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ibp_compress with
 * the workspace taken from a fixed array inside the library instead of an argument.
 * The array is IBP_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from the
 * library's first such call on that GPU until the process ends; the call itself
 * allocates nothing.  Inputs up to IBP_NOALLOC_SCRATCH_BYTES of compression
 * workspace (ibp_compress_workspace_bytes(n, S) <= the limit: about 2 * 10^9 chunks
 * at S = 256) are accepted; larger ones return IBP_ERR_CAPACITY before any launch.
 *   Uses the GPU that is current on the calling thread; hip_stream must belong to it.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on one
 *   GPU (other streams, other threads) race and may corrupt each other's output;
 *   calls on one stream are ordered and safe.  The array is cleared by a kernel at
 *   the start of each call, so no state carries from one call to the next.
 *   Other arguments, outputs and errors as ibp_compress; IBP_ERR_DEVICE also when the
 *   array's address cannot be resolved.
 */
#define IBP_NOALLOC_SCRATCH_BYTES (8ull << 20)
IBP_API int ibp_compress_noalloc(const ibp_meta_t *meta, const void *d_in, uint64_t n_bytes, uint32_t S,
                                 void *d_stream, uint64_t stream_capacity, uint64_t *d_offsets,
                                 uint32_t *d_err_word, void *hip_stream);

/*
 * Step 3 -- decompression, device-resident ("Algoritmo Core", Decompressione).
 *   stream_in: compressed stream (device, or pinned host memory), aligned to 16,
 *     readable for stream_bytes bytes.
 *   d_offsets: nseg + 1 bit offsets (device), nseg = ceil(n_chunks / S).
 *   d_out: n_chunks * W/8 bytes (device, aligned to W/8).
 *   A segment whose offsets are inconsistent is not decoded and sets
 *   IBP_DEVERR_CORRUPT; no read goes outside [stream_in, stream_in + stream_bytes).
 */
IBP_API int ibp_decompress(const ibp_meta_t *meta, const void *stream_in, uint64_t stream_bytes,
                           const uint64_t *d_offsets, uint64_t n_chunks, uint32_t S, void *d_out,
                           uint32_t *d_err_word, void *hip_stream);

/*
 * Step 3 on a gather ("Integrazione del Sistema", PCIe Transfer Compression):
 * row j of d_out (S chunks) = segment d_ids[j] of a stream of n_segments full
 * segments of S chunks.  stream_in is normally pinned host memory, read by the
 * kernel over PCIe without a staging copy; device memory works too.
 *   d_ids: n_ids int64 segment ids (device).  Duplicates are decoded again.
 *   d_out: n_ids * S * W/8 bytes (device).  A row whose id is out of range is
 *   left untouched and sets IBP_DEVERR_BAD_ID.
 */
IBP_API int ibp_decompress_gather(const ibp_meta_t *meta, const void *stream_in, uint64_t stream_bytes,
                                  const uint64_t *d_offsets, uint64_t n_segments, uint32_t S,
                                  const int64_t *d_ids, uint64_t n_ids, void *d_out,
                                  uint32_t *d_err_word, void *hip_stream);

/*
 * Baseline for the measurements, not part of the codec: the uncompressed
 * transfer that IBP replaces (the page's "Risultati" compare against it).
 * Row j of d_out = row d_ids[j] of a table of n_rows rows of row_bytes bytes at
 * src (pinned host memory or device memory, aligned to 16); row_bytes % 16 == 0.
 * Out-of-range ids leave the row untouched and set IBP_DEVERR_BAD_ID.  n_rows == 0
 * with n_ids > 0, or a byte count beyond 64 bits, is IBP_ERR_SIZE.
 */
IBP_API int ibp_gather_raw(const void *src, uint64_t row_bytes, uint64_t n_rows, const int64_t *d_ids,
                           uint64_t n_ids, void *d_out, uint32_t *d_err_word, void *hip_stream);

/*
 * Fixed-slot layout ("Integrazione del Sistema", PCIe Transfer Compression: tensors
 * compressed in place in fixed-size buffers of which only the compressed part is
 * read, with a bit vector in GPU memory marking the compressed ones).
 *   Row r (S chunks, row_bytes = S*W/8, which must be a multiple of 16) owns bytes
 *   [r*row_bytes, (r+1)*row_bytes) of `slots`.  If the row's segment encoding
 *   (S participation bits, then the payloads: the same bits as a segment of the
 *   packed stream) is shorter than S*W bits, the slot holds those bits from its bit
 *   0 and bit r%64 of d_flags[r/64] is 1; otherwise the slot holds the raw row and
 *   the bit is 0.  The used length of a compressed slot follows from its header.
 */

/* 64-bit flag words for n_rows rows: ceil(n_rows / 64). */
IBP_API uint64_t ibp_slot_flag_words(uint64_t n_rows);

/* Compress n_rows rows of d_in (device or pinned host memory, aligned to 16) into
 * their slots (device or pinned host memory, aligned to 16, slots_bytes >=
 * n_rows*row_bytes).  d_flags (device memory, ibp_slot_flag_words(n_rows) words)
 * is cleared and filled.  Slot bytes after a compressed row's last 16-byte block
 * are not written.  Asynchronous. */
IBP_API int ibp_compress_slots(const ibp_meta_t *meta, const void *d_in, uint64_t n_rows, uint32_t S,
                               void *slots, uint64_t slots_bytes, uint64_t *d_flags, uint32_t *d_err_word,
                               void *hip_stream);

/* Row j of d_out = row d_ids[j] of a slot table of n_rows rows (slots in pinned
 * host memory, read zero-copy, or device memory).  Only the used part of a
 * compressed slot is read: a first round reads as much as the shortest
 * compressed row can use (its header included), in whole 128-byte lines when
 * row_bytes is a multiple of 128; a longer row's rest follows in a second round.
 * Out-of-range ids leave the row untouched and set IBP_DEVERR_BAD_ID.
 * Asynchronous. */
IBP_API int ibp_decompress_gather_slots(const ibp_meta_t *meta, const void *slots, uint64_t slots_bytes,
                                        uint64_t n_rows, uint32_t S, const uint64_t *d_flags,
                                        const int64_t *d_ids, uint64_t n_ids, void *d_out,
                                        uint32_t *d_err_word, void *hip_stream);

/*
 * Position-dependent metadata ("Algoritmo Core", Preprocessing: metadata of fixed
 * size, of the order of kilobytes).  Chunk position i of every segment (row of S
 * chunks), i < S, has its own Mask_i and Bitval_i; the stream layout is that of
 * ibp_compress, a matching chunk at position i keeping its W - popcount(Mask_i)
 * bits outside Mask_i.  A short last segment uses positions 0 .. m-1.
 */
typedef struct {
  uint32_t W;             /* chunk width in bits: 16, 32 or 64 */
  uint32_t S;             /* positions = chunks per segment, 1..IBP_MAX_S */
  const uint64_t *mask;   /* device memory, S words: Mask_i (bits at or above W are ignored) */
  const uint64_t *bitval; /* device memory, S words: Bitval_i (bits outside Mask_i are ignored) */
} ibp_pos_meta_t;

/* Workspace for ibp_build_metadata_pos: 8 * S * W bytes (the per-position counts). */
IBP_API uint64_t ibp_metadata_pos_workspace_bytes(uint32_t S, uint32_t W);

/* Step 1 per position: d_samples holds n_rows sample rows of S chunks (device,
 * aligned to W/8); Mask_i / Bitval_i follow the rule of ibp_build_metadata over
 * the i-th chunk of every row (N = n_rows) and are written to d_mask[i] /
 * d_bitval[i] (device, S words each).  counts_out (host, optional): S*W uint64,
 * counts_out[i*W + b] = rows whose chunk i has bit b set; when given, the call
 * waits for hip_stream, otherwise it is asynchronous. */
IBP_API int ibp_build_metadata_pos(const void *d_samples, uint64_t n_rows, uint32_t S, uint32_t W, double T,
                                   uint64_t *d_mask, uint64_t *d_bitval, uint64_t *counts_out, void *d_workspace,
                                   uint64_t workspace_bytes, void *hip_stream);

/* Step 2 with position-dependent metadata; S = meta->S.  Arguments, sizes,
 * workspace (ibp_compress_workspace_bytes(n, S)) and errors as ibp_compress. */
IBP_API int ibp_compress_pos(const ibp_pos_meta_t *meta, const void *d_in, uint64_t n_bytes, void *d_stream,
                             uint64_t stream_capacity, uint64_t *d_offsets, void *d_workspace,
                             uint64_t workspace_bytes, uint32_t *d_err_word, void *hip_stream);

/* Step 3 with position-dependent metadata; S = meta->S.  Arguments and errors as
 * ibp_decompress. */
IBP_API int ibp_decompress_pos(const ibp_pos_meta_t *meta, const void *stream_in, uint64_t stream_bytes,
                               const uint64_t *d_offsets, uint64_t n_chunks, void *d_out, uint32_t *d_err_word,
                               void *hip_stream);

/*
 * Comparison codec, not IBP: exponent coding of BF16 tensors as on the page
 * "ZipCCL: Efficient Lossless Data Compression of Communication Collectives for
 * Accelerating LLM Training" (section 2, Metodologia, A and B), on one GPU.
 *   Element i (BF16 word u) -> sign-mantissa byte sm[i] = (u >> 8 & 0x80) | (u & 0x7F)
 *   and exponent e = (u >> 7) & 0xFF.  If e == table[k] the element's code is k + 1,
 *   otherwise 0 and e is appended to the escape array (element order).
 *   Blocks of 4096 elements; block j keeps its codes as three planes of 512 bytes
 *   at d_codes + j*1536 + p*512 (bit t of plane p = bit p of element t's code,
 *   LSB-first bytes; bits past the last element are 0).  d_eoff[j] = escapes
 *   before block j, d_eoff[nblk] = total escapes.
 *   table: host, 7 distinct exponents (codes 1..7).
 */

/* The 7 exponents of largest mass under N(0, sigma^2) (exponent e covers
 * 2^(e-127) <= |x| < 2^(e-126); e = 0 covers |x| < 2^-126; e = 255 none), in
 * decreasing mass order, equal masses by smaller exponent: 7 bytes to table_out. */
IBP_API int ibp_zip_table_from_sigma(double sigma, uint8_t *table_out);

/* ceil(n / 4096); code plane bytes 1536 * blocks; compression workspace 8 bytes plus
 * 8 per look-back status word (16 per line over 2^k lines, 16 * 2^k >= ceil(blocks / 4)). */
IBP_API uint64_t ibp_zip_blocks(uint64_t n);
IBP_API uint64_t ibp_zip_codes_bytes(uint64_t n);
IBP_API uint64_t ibp_zip_workspace_bytes(uint64_t n);

/* Compress n BF16 words (d_in, device, aligned to 16).  d_sm: n bytes (aligned to
 * 8); d_codes: ibp_zip_codes_bytes(n); d_esc: esc_capacity >= n bytes; d_eoff:
 * blocks + 1 words; d_workspace: ibp_zip_workspace_bytes(n).  One pass: each
 * block finds its first escape by a decoupled look-back over the blocks (bounded;
 * IBP_DEVERR_TIMEOUT on give-up).  Asynchronous. */
IBP_API int ibp_zip_compress(const uint8_t *table, const void *d_in, uint64_t n, uint8_t *d_sm, uint8_t *d_codes,
                             uint8_t *d_esc, uint64_t esc_capacity, uint64_t *d_eoff, void *d_workspace,
                             uint64_t workspace_bytes, uint32_t *d_err_word, void *hip_stream);

/* Decompress n BF16 words into d_out (device, aligned to 16).  esc_bytes: readable
 * escape bytes.  A block whose escape count disagrees with d_eoff, or whose
 * escapes lie past esc_bytes, is not decoded and sets IBP_DEVERR_CORRUPT. */
IBP_API int ibp_zip_decompress(const uint8_t *table, const uint8_t *d_sm, const uint8_t *d_codes,
                               const uint8_t *d_esc, uint64_t esc_bytes, const uint64_t *d_eoff, uint64_t n,
                               void *d_out, uint32_t *d_err_word, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* IBP_H */
