/*
 * ec.h - lossless fixed-codebook entropy coding of 8-bit e4m3 tensor bytes
 *        on AMD Instinct MI355X (gfx950).  C ABI, version 1.
 *
 * Codecs
 *   QLC          Quad Length Codes: "Quad Length Codes for Lossless
 *                Compression of e4m3", section 2.  Symbols ranked by
 *                decreasing probability, 8 areas chosen by a 3-bit prefix,
 *                one code length per area, 256-entry LUT encode, prefix ->
 *                length decode.
 *   Huffman      single-stage Huffman: "Single-Stage Huffman Encoder for ML
 *                Compression", TL;DR and abstract.  One fixed codebook built
 *                from the average distribution of earlier batches, stored on
 *                the device, never sent with the data.
 *   Exp-Golomb   order-k Exp-Golomb on the QLC rank, the universal-code
 *                baseline of the QLC page, section 1.
 *
 * Memory and ownership
 *   - Every pointer named d_* is device memory that the caller allocates and
 *     owns.  Input and output buffers must be 16-byte aligned.
 *   - ec_codebook is an opaque, library-owned handle made by a *_build_*
 *     function and released with ec_codebook_free.  Its device tables are
 *     allocated on the current device at its first GPU use and freed with
 *     the handle.
 *   - The library keeps four scratch buffers per device and stream,
 *     allocated with hipMalloc on first use, grown by doubling and kept
 *     until the process ends: the encoder's chunk sizes (4 bytes per chunk
 *     of a launch), the histogram's partial counts (1 KiB per partial row),
 *     and the BF16 encoder's escape counts and staged escapes.  Calls on one
 *     stream run in order and share them; calls on different streams do not.
 *     An allocation or growth inside an asynchronous entry point synchronises
 *     the device implicitly and cannot happen under stream capture:
 *     entropy_encode_noalloc takes none.  A stream destroyed while its work
 *     runs and a new stream that gets the same handle share the buffers:
 *     let the old work finish first.
 *   - Device codebook tables (the *_device functions) live in caller-owned
 *     device memory: n_seg consecutive tables of ec_device_codebook_bytes()
 *     bytes each, 16-byte aligned.
 *
 * Errors
 *   - Functions return an ec_error code for argument, allocation and launch
 *     problems; GPU work is enqueued asynchronously on the given stream.
 *   - Data-dependent problems found on the device are OR-ed into a caller
 *     zeroed status word (EC_S_* bits), readable after the stream syncs.
 *     When a status bit is set, the output contents are unspecified.
 *
 * Stream container (this library's own; the pages fix the codes, not a byte
 * format).  All integers little-endian.
 *   offset 0   u32 magic 0x53384345 ("EC8S")    4  u16 version 1
 *          6   u8  codec (ec_codec)             7  u8  flags (bit 0: code lengths embedded)
 *          8   u64 n_symbols                   16  u32 chunk_symbols C (multiple of 256)
 *         20   u32 n_chunks = ceil(n / C)      24  u64 payload_offset (multiple of 256)
 *         32   u64 payload_bytes               40  u64 codebook_id
 *         48   16 zero bytes
 *         64   u64 chunk_off[n_chunks + 1]: byte offset of each chunk in the
 *              payload; each a multiple of 16
 *              u32 sub_end[n_chunks][C / 256]: bit offset, from the chunk's
 *              start, where each 256-symbol sub-chunk ends; sub-chunks past
 *              n hold the chunk's total bit count
 *              u8 code_len[256] (only with flags bit 0)
 *              zero bytes up to payload_offset
 *   payload: chunk c occupies [chunk_off[c], chunk_off[c+1]); its bits form
 *   32-bit little-endian words, bit i of the chunk being bit (31 - i % 32)
 *   of word i / 32; codes are written most significant bit first in symbol
 *   order; bits after the last code up to the 16-byte boundary are zero.
 */
#ifndef EC_H
#define EC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of every int-returning function. */
typedef enum ec_error {
    EC_OK = 0,
    EC_E_INVAL = 1,        /* bad argument: NULL, size, alignment, layout */
    EC_E_UNSUPPORTED = 2,  /* e.g. a Huffman code longer than EC_MAX_CODE_LEN bits */
    EC_E_NOMEM = 3,        /* host or device allocation failed */
    EC_E_HIP = 4,          /* a HIP runtime call or kernel launch failed */
    EC_E_CAPACITY = 5      /* out_cap cannot even hold the header and index */
} ec_error;

/* Device status bits (OR-ed into *d_status). */
#define EC_S_CAPACITY 0x1u          /* encoded stream longer than out_cap; nothing past out_cap written */
#define EC_S_CORRUPT 0x2u           /* payload or index does not decode consistently */
#define EC_S_BAD_HEADER 0x4u        /* magic, version, sizes or layout wrong */
#define EC_S_CODEBOOK_MISMATCH 0x8u /* stream made with another codebook or codec */
#define EC_S_BAD_CODEBOOK 0x10u     /* device codebook build: a code would exceed EC_MAX_CODE_LEN
                                       bits (or a count is 2^55 or more); the table is unusable
                                       (codec 0) and encodes that use it set this bit too */

typedef enum ec_codec {
    EC_CODEC_QLC = 1,
    EC_CODEC_HUFFMAN = 2,
    EC_CODEC_EXP_GOLOMB = 3
} ec_codec;

#define EC_MAX_CODE_LEN 40      /* longest Huffman code the GPU path supports */
#define EC_MAX_BATCH 128        /* segments per batch call */

typedef struct ec_codebook ec_codebook;

/* ---------------------------------------------------------------------------
 * Codebook builders (host only, no GPU needed).
 * ------------------------------------------------------------------------- */

/*
 * Quad Length Code ("Quad Length Codes for Lossless Compression of e4m3",
 * section 2: areas, LUT encode; section 3: adapted area sizes).
 *   counts[256]      byte frequencies; symbols are ranked by decreasing count,
 *                    equal counts by increasing byte value
 *   area_size[8]     symbols in area a = 0..7; must sum to 256
 *   suffix_bits[8]   bits after the 3-bit prefix in area a, 0..8, with
 *                    area_size[a] <= 2^suffix_bits[a]
 * Rank r in area a is coded as a (3 bits) then r - first_rank(a)
 * (suffix_bits[a] bits).  Base scheme: sizes 8,8,8,8,8,16,32,168 with suffix
 * bits 3,3,3,3,3,4,5,8.  Returns EC_E_INVAL on a bad layout.
 */
int qlc_build_codebook(const uint64_t counts[256], const uint16_t area_size[8],
                       const uint8_t suffix_bits[8], ec_codebook **out);

/*
 * QLC area layout with the fewest payload bits for these counts (QLC page,
 * section 2: the symbols per area and the code lengths adapt to the
 * distribution while at most four distinct lengths remain; section 5: a
 * mathematical optimisation of both is the authors' next step).
 *   counts[256]      byte frequencies, ranked as for qlc_build_codebook
 *   max_lengths      1..8: most distinct code lengths among non-empty areas
 *                    (4 keeps the quad-length property; 8 leaves it free)
 *   area_size[8], suffix_bits[8]  out: a layout for qlc_build_codebook
 * Minimises sum over ranks of count x (3 + suffix width of the rank's area).
 * Of the cheapest layouts it returns the one whose non-empty areas have
 * non-decreasing widths, all full (2^width symbols) but the last, followed
 * by unused areas (size 0, width 0), with the lexicographically smallest
 * width sequence.  Host memory only; EC_E_INVAL on NULL pointers or
 * max_lengths outside 1..8.
 */
int qlc_optimal_area_layout(const uint64_t counts[256], uint32_t max_lengths, uint16_t area_size[8],
                            uint8_t suffix_bits[8]);

/*
 * Huffman codebook ("Single-Stage Huffman Encoder for ML Compression",
 * abstract and method steps 2-3: one tree built from the average
 * distribution of earlier batches).
 *   counts[256]  summed byte counts of the calibration data (for shards of
 *                equal size this is proportional to their average PMF).
 *                Every symbol is weighted counts[s] + 1 so that symbols not
 *                seen in calibration still get a code.  Counts must be
 *                below 2^55 (EC_E_INVAL otherwise).
 * The tree merges the two lightest nodes, ties ordered by (weight, leaves
 * before internal nodes, byte value / creation order); codes are canonical
 * in (length, byte) order.  EC_E_UNSUPPORTED if a code exceeds
 * EC_MAX_CODE_LEN bits.
 */
int huff_build_codebook(const uint64_t counts[256], ec_codebook **out);

/*
 * Huffman codebook from 256 code lengths (as embedded in a stream by the
 * three-stage path, single-stage Huffman page, abstract: the codebook
 * transmitted with the data).  Lengths must form a complete prefix code
 * (Kraft sum exactly 1) of at most EC_MAX_CODE_LEN bits, else EC_E_INVAL.
 */
int huff_build_codebook_from_lengths(const uint8_t code_len[256], ec_codebook **out);

/*
 * Exp-Golomb on rank (QLC page, section 1: universal codes such as
 * Exponential-Golomb).  Symbols ranked as for QLC; rank r is coded with
 * order k: v = r + 2^k, m = floor(log2 v), m - k zeros then v in m + 1 bits.
 *   k in 0..8, or -1 to pick the k that minimises sum(counts * length),
 *   ties to the smaller k.
 */
int eg_build_codebook(const uint64_t counts[256], int k, ec_codebook **out);

/*
 * Huffman code lengths for n (2..256) positive weights, same tree rule as
 * huff_build_codebook but without the +1 smoothing and without a length
 * cap.  len_out[n].
 */
int huff_code_lengths(const uint64_t *weights, uint32_t n, uint8_t *len_out);

/*
 * Describe a codebook.  Any output pointer may be NULL.
 *   code[256]         code value of each byte (len low bits, MSB first)
 *   code_len[256]     code length of each byte in bits
 *   rank_to_sym[256]  QLC / Exp-Golomb rank order (zeros for Huffman)
 *   eg_k              Exp-Golomb order (-1 for other codecs)
 */
int ec_codebook_info(const ec_codebook *cb, uint32_t *codec, uint32_t *max_len,
                     uint64_t *codebook_id, uint8_t code_len[256], uint64_t code[256],
                     uint8_t rank_to_sym[256], int32_t *eg_k);

void ec_codebook_free(ec_codebook *cb);

/* ---------------------------------------------------------------------------
 * Stream sizing (host only).
 * ------------------------------------------------------------------------- */

/* Bytes before the payload: header + index (+256 with embedded lengths),
 * rounded up to 256.  0 on bad arguments. */
uint64_t entropy_index_bytes(uint64_t n, uint32_t chunk_symbols, uint32_t embed_lengths);

/* Largest possible stream for n symbols with this codebook.  0 on bad args. */
uint64_t entropy_max_encoded_bytes(const ec_codebook *cb, uint64_t n, uint32_t chunk_symbols,
                                   uint32_t embed_lengths);

/* ---------------------------------------------------------------------------
 * GPU operations: asynchronous on `stream` (0 = the null stream).
 * ------------------------------------------------------------------------- */

/*
 * Encode n bytes (QLC page, section 2: "the encoder looks up the code in the
 * table"; single-stage Huffman page, method step 4: encode directly with the
 * precomputed codebook).
 *   d_in           n input bytes
 *   chunk_symbols  C: multiple of 256, 256..65536; chunks are coded
 *                  independently and sub-chunk offsets every 256 symbols let
 *                  the decoder start 256-symbol runs in parallel
 *   d_out          out_cap bytes; receives the stream
 *   d_out_len      device u64: the stream length, also when it exceeds
 *                  out_cap (EC_S_CAPACITY is then set and nothing past
 *                  out_cap is written)
 *   d_status       device u32, caller-zeroed; may be NULL
 * Returns EC_E_CAPACITY if out_cap < entropy_index_bytes(n, C, 0).
 */
int entropy_encode(const ec_codebook *cb, const uint8_t *d_in, uint64_t n, uint32_t chunk_symbols,
                   uint8_t *d_out, uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status,
                   hipStream_t stream);

/*
 * entropy_encode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, same stream, but no allocation of any kind.
 *   - The codebook's device tables must already be on the current device:
 *     any earlier GPU call with this codebook on this device (for example
 *     one entropy_encode) puts them there.  EC_E_INVAL otherwise.
 *   - The per-chunk sizes go to a fixed library array on each device, of
 *     65536 entries: at most 65536 chunks a call (ceil(n / chunk_symbols)),
 *     EC_E_UNSUPPORTED beyond.  The array keeps the last call's contents;
 *     nothing in it needs clearing (each call writes every entry it reads).
 *   - Every call on one device shares that array: two of these calls that
 *     overlap in time on one device (different streams) race.  Order them.
 */
int entropy_encode_noalloc(const ec_codebook *cb, const uint8_t *d_in, uint64_t n, uint32_t chunk_symbols,
                           uint8_t *d_out, uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status,
                           hipStream_t stream);

/*
 * Decode a stream made by entropy_encode with the same codebook (QLC page,
 * section 2: read the 3-bit area code, which fixes the length, then the
 * rest; area offset; second LUT.  Huffman: two-level table lookup instead of
 * a bit-serial tree walk).
 *   d_in    the stream; in_len = bytes readable at d_in (>= stream length)
 *   d_out   n bytes; n must equal the stream's n_symbols
 *   d_status  device u32, caller-zeroed; may be NULL.  Header, codebook and
 *           consistency failures set EC_S_* bits; decoding never reads
 *           outside [d_in, d_in + in_len).
 */
int entropy_decode(const ec_codebook *cb, const uint8_t *d_in, uint64_t in_len,
                   uint8_t *d_out, uint64_t n, uint32_t *d_status, hipStream_t stream);

/*
 * entropy_encode with the chunk sizes already made by byte_histogram_sized
 * for this codebook, input and chunk_symbols (its d_sizes row for cb): no
 * sizing pass, the input is read once.  The stream is the one
 * entropy_encode makes.
 *   d_sizes   device u32[ceil(n / chunk_symbols)], 4-byte aligned; read only
 *   Codebooks whose codes exceed 26 bits, or chunks of more than 16384
 *   symbols: EC_E_UNSUPPORTED.  A chunk whose size differs from the one its
 *   packer computes (sizes made for another codebook or input) sets
 *   EC_S_CODEBOOK_MISMATCH; the stream is then unusable.
 */
int entropy_encode_sized(const ec_codebook *cb, const uint8_t *d_in, uint64_t n, uint32_t chunk_symbols,
                         const uint32_t *d_sizes, uint8_t *d_out, uint64_t out_cap, uint64_t *d_out_len,
                         uint32_t *d_status, hipStream_t stream);

/*
 * Encode n_seg (1..EC_MAX_BATCH) segments of seg_n bytes in one launch.
 * Segment s is read at d_in + s * in_stride and coded with cbs[s] (all
 * entries may be the same handle: single-stage path; or one per shard:
 * three-stage path, single-stage Huffman page, abstract).  Its stream goes
 * to d_out + s * out_stride (out_stride bytes of capacity), its length to
 * d_out_len[s], its status bits to d_status[s] (may be NULL).
 * embed_lengths = 1 stores the 256 code lengths in each stream (the
 * "codebook transmitted with the data" of the three-stage design).
 */
int entropy_encode_batch(const ec_codebook *const *cbs, uint32_t n_seg, const uint8_t *d_in,
                         uint64_t seg_n, uint64_t in_stride, uint32_t chunk_symbols,
                         uint32_t embed_lengths, uint8_t *d_out, uint64_t out_stride,
                         uint64_t *d_out_len, uint32_t *d_status, hipStream_t stream);

/*
 * entropy_encode_batch with caller-made chunk sizes, as entropy_encode_sized:
 * d_sizes[s][c] is the size of segment s's chunk c under cbs[s] (with one
 * codebook for every segment, its d_sizes block from byte_histogram_sized).
 */
int entropy_encode_batch_sized(const ec_codebook *const *cbs, uint32_t n_seg, const uint8_t *d_in,
                               uint64_t seg_n, uint64_t in_stride, uint32_t chunk_symbols,
                               uint32_t embed_lengths, const uint32_t *d_sizes, uint8_t *d_out,
                               uint64_t out_stride, uint64_t *d_out_len, uint32_t *d_status,
                               hipStream_t stream);

/*
 * The receiving side of entropy_encode_batch: decode n_seg (1..EC_MAX_BATCH)
 * streams in one launch (single-stage Huffman page, methodology step 4 and
 * "Practical Implications": every accelerator holds the same precomputed
 * codebook, so a receiver decodes each shard it gets with cbs[s] and
 * nothing else; the three-stage path passes each shard's own codebook).
 * Stream s is read at d_in + s * in_stride (in_stride readable bytes, at
 * least its length); its seg_n decoded bytes go to d_out + s * out_stride.
 * cbs[s] must be the codebook stream s was coded with (same codec and id,
 * else EC_S_CODEBOOK_MISMATCH in d_status[s]).  d_status: device u32[n_seg],
 * caller-zeroed, or NULL; per-stream bits as for entropy_decode.  No read
 * leaves [d_in + s * in_stride, + in_stride) for stream s.
 */
int entropy_decode_batch(const ec_codebook *const *cbs, uint32_t n_seg, const uint8_t *d_in,
                         uint64_t in_stride, uint8_t *d_out, uint64_t seg_n, uint64_t out_stride,
                         uint32_t *d_status, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Device-resident codebooks: the three-stage path without a host round trip
 * (single-stage Huffman page, abstract: frequency analysis, codebook
 * generation, encoding with the shard's own codebook, which travels with the
 * data).  Histogram rows -> huff_build_codebooks_device -> the *_device
 * encode and decode, all enqueued on one stream.
 * ------------------------------------------------------------------------- */

/* Bytes of one device codebook table (a multiple of 16). */
uint64_t ec_device_codebook_bytes(void);

/*
 * Build one Huffman codebook per segment on the GPU from d_counts[s * 256 + b]
 * (as written by byte_histogram), with exactly the rule and the tables of
 * huff_build_codebook (weights counts + 1, the same merge order and tie rule,
 * canonical codes, the same codebook id).
 *   n_seg     1..65535
 *   d_tables  n_seg * ec_device_codebook_bytes() bytes, 16-byte aligned;
 *             overwritten
 *   d_status  device u32[n_seg], caller-zeroed, or NULL: EC_S_BAD_CODEBOOK
 *             when the segment's code would need more than EC_MAX_CODE_LEN
 *             bits or a count is 2^55 or more (its table is then unusable:
 *             codec 0, all zero).
 */
int huff_build_codebooks_device(const uint64_t *d_counts, uint32_t n_seg, void *d_tables, uint32_t *d_status,
                                hipStream_t stream);

/*
 * The receiving side: rebuild, on the GPU, the tables of the Huffman
 * codebook each stream carries (the 256 code lengths that
 * entropy_encode_batch[_device] embeds with embed_lengths = 1), so that a
 * decoder needs nothing but the stream (single-stage Huffman page, abstract:
 * the codebook transmitted with the data).  The tables equal those of
 * huff_build_codebook_from_lengths.
 *   d_in       n_seg streams at d_in + s * in_stride (in_len readable bytes
 *              each; in_stride a multiple of 16 and >= in_len when n_seg > 1)
 *   d_tables   as for huff_build_codebooks_device
 *   d_status   device u32[n_seg], caller-zeroed, or NULL:
 *              EC_S_BAD_HEADER   not a Huffman stream with embedded lengths,
 *                                or its index does not fit in in_len;
 *              EC_S_BAD_CODEBOOK the lengths are not a complete prefix code
 *                                of 1..EC_MAX_CODE_LEN-bit codes.
 *              Either way the segment's table is unusable (codec 0).
 */
int huff_tables_from_streams_device(const uint8_t *d_in, uint64_t in_stride, uint64_t in_len, uint32_t n_seg,
                                    void *d_tables, uint32_t *d_status, hipStream_t stream);

/*
 * Copy a host-built codebook's table, in the device table format, to host
 * memory `table` (ec_device_codebook_bytes() bytes).  Uploaded into a device
 * table array it serves the *_device functions like a device-built one.
 */
int ec_codebook_export(const ec_codebook *cb, void *table);

/*
 * Capacity per stream that always suffices when segment s is coded with a
 * Huffman codebook built from its own byte histogram (three-stage path):
 * such a code never spends more than 8 bits a symbol on the segment as a
 * whole (a Huffman code is no longer than the 8-bit fixed code on its
 * weights counts + 1, and 256 complete-code lengths sum to at least 2048),
 * plus at most 16 bytes of padding per chunk.  0 on bad arguments.
 */
uint64_t entropy_own_max_encoded_bytes(uint64_t n, uint32_t chunk_symbols, uint32_t embed_lengths);

/*
 * entropy_encode_batch with the codebooks in device memory: segment s uses
 * the table at d_tables + s * ec_device_codebook_bytes().  n_seg 1..
 * EC_MAX_BATCH.  The host does not read the tables, so it cannot size
 * anything from them: chunks whose table has codes longer than 26 bits are
 * packed by the general row-by-row packer; a stream longer than out_stride
 * sets EC_S_CAPACITY (see entropy_own_max_encoded_bytes).  A table marked
 * unusable sets EC_S_BAD_CODEBOOK.
 */
int entropy_encode_batch_device(const void *d_tables, uint32_t n_seg, const uint8_t *d_in, uint64_t seg_n,
                                uint64_t in_stride, uint32_t chunk_symbols, uint32_t embed_lengths,
                                uint8_t *d_out, uint64_t out_stride, uint64_t *d_out_len, uint32_t *d_status,
                                hipStream_t stream);

/*
 * entropy_decode_batch with the codebooks in device memory (as for
 * entropy_encode_batch_device); `codec` is the codec of every table
 * (EC_CODEC_*).  A stream whose header names another codec or codebook id
 * than its table sets EC_S_CODEBOOK_MISMATCH.
 */
int entropy_decode_batch_device(const void *d_tables, uint32_t codec, uint32_t n_seg, const uint8_t *d_in,
                                uint64_t in_stride, uint8_t *d_out, uint64_t seg_n, uint64_t out_stride,
                                uint32_t *d_status, hipStream_t stream);

/*
 * Byte histogram of n_seg segments (single-stage Huffman page, method step
 * 1 and the abstract's "frequency analysis" stage):
 * d_counts[s * 256 + b] = number of bytes equal to b in segment s, read at
 * d_in + s * in_stride (seg_n bytes; any alignment).  d_counts is
 * overwritten.
 */
int byte_histogram(const uint8_t *d_in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride,
                   uint64_t *d_counts, hipStream_t stream);

/*
 * byte_histogram that, in the same pass over the input, also sizes the
 * chunks an encode of each segment would make with each of n_cb (1..4)
 * codebooks.  The single-stage design fixes the codebooks before the data
 * is seen (single-stage Huffman page, TL;DR and method steps 2-4; QLC page,
 * section 2: fixed tables), so the pass that gathers the statistics can also
 * add up the code lengths; entropy_encode_sized then reads the input once.
 *   d_in           16-byte aligned; in_stride a multiple of 16 (n_seg > 1)
 *   chunk_symbols  a power of two, 256..16384 (32768 and 65536 too when the
 *                  launch is large); every seg_n a multiple of 16.  Other
 *                  shapes: EC_E_UNSUPPORTED (use byte_histogram and
 *                  entropy_encode).
 *   d_sizes        device u32[n_cb][n_seg][ceil(seg_n / chunk_symbols)]:
 *                  chunk sizes in 16-byte units, overwritten
 * d_counts as for byte_histogram.
 */
int byte_histogram_sized(const uint8_t *d_in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride,
                         uint64_t *d_counts, const ec_codebook *const *cbs, uint32_t n_cb,
                         uint32_t chunk_symbols, uint32_t *d_sizes, hipStream_t stream);

/*
 * Average PMF of n_seg count rows (single-stage Huffman page, TL;DR and
 * method step 2): d_pmf[b] = (1/S) sum_s counts[s][b] / sum_b' counts[s][b'],
 * computed in fp32.  Rows with no counts contribute zero.
 */
int pmf_average(const uint64_t *d_counts, uint32_t n_seg, float *d_pmf, hipStream_t stream);

/*
 * KL divergence of each row from a reference (single-stage Huffman page,
 * TL;DR and figure 3: KL of shard PMFs from the average PMF), in bits:
 * d_kl_bits[s] = sum_{P_b > 0} P_b log2(P_b / Q_b), P the row's PMF,
 * Q_b = (q_b + q_add) / sum(q + q_add).  fp32 result from a
 * cancellation-free form; +inf when some Q_b = 0 < P_b.
 */
int pmf_kl(const uint64_t *d_p, uint32_t n_seg, const uint64_t *d_q, uint32_t q_add,
           float *d_kl_bits, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Exponent coding of BF16 tensors ("ZipCCL: Efficient Lossless Data
 * Compression of Communication Collectives for Accelerating LLM Training",
 * methodology A-C).  A value splits into its sign-and-mantissa byte and its
 * 8-bit exponent; the seven exponents of a table get the 3-bit codes 1..7,
 * any other exponent code 0 and a place in an escape array.  Stream layout
 * (little-endian): 64-byte header (magic "EB16", version 1, n, chunk values,
 * chunk count, the 7 table exponents, escape count, section offsets); u64
 * esc_off[n_chunks + 1] (escapes before each chunk); zero fill to 256; n
 * sign-mantissa bytes (sign << 7 | mantissa); zero fill to 16; three code
 * planes (bit k of value i's code is bit i & 7 of byte i >> 3 of plane k),
 * each zero-padded to a multiple of 16 bytes; the escaped exponents in value
 * order.
 * ------------------------------------------------------------------------- */

/* The seven exponents with the largest counts (counts[e] for exponent e),
 * most frequent first, equal counts to the smaller exponent.  Host memory. */
int bf16_exp_table_from_counts(const uint64_t counts[256], uint8_t table[7]);

/* The table predicted from the standard deviation alone (ZipCCL page,
 * methodology A: near-Gaussian tensors): the seven exponents whose octaves
 * [2^(e-127), 2^(e-126)) hold the most N(0, sigma^2) mass, largest first,
 * equal masses to the smaller exponent.  EC_E_INVAL unless sigma > 0. */
int bf16_exp_table_from_sigma(double sigma, uint8_t table[7]);

/* Bytes that always hold the stream of n values (every exponent escaped);
 * 0 on bad arguments.  chunk: values per chunk, a multiple of 2048 from
 * 2048 to 2^20. */
uint64_t bf16_exp_max_encoded_bytes(uint64_t n, uint32_t chunk);

/*
 * Encode n BF16 values (d_in: device, 16-byte aligned, bit patterns) with
 * table[7] (seven distinct exponents, host memory) in chunks of `chunk`
 * values into d_out (device, 16-byte aligned, out_cap bytes).  The stream
 * length is stored in device *d_out_len.  At most 8192 chunks a stream
 * (EC_E_UNSUPPORTED beyond).  EC_E_CAPACITY when out_cap cannot hold the
 * sections before the escapes; when the escapes do not fit, nothing is
 * written past out_cap, *d_out_len still gets the needed length and
 * EC_S_CAPACITY is OR-ed into *d_status (device u32 or NULL).  Asynchronous
 * on `stream`; uses library scratch of the device and stream (an escape
 * count per chunk and a staging area of chunk bytes per chunk).
 */
int bf16_exp_encode(const uint8_t table[7], const uint16_t *d_in, uint64_t n, uint32_t chunk, uint8_t *d_out,
                    uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status, hipStream_t stream);

/*
 * Decode a stream of bf16_exp_encode (d_in: device, 16-byte aligned, in_len
 * readable bytes) into n BF16 values at d_out (device, 16-byte aligned).
 * The table and chunk size come from the stream's header.  Into *d_status:
 * EC_S_BAD_HEADER (wrong magic or version, n differs, sections not where
 * the layout puts them or beyond in_len) or EC_S_CORRUPT (escape index
 * inconsistent with the code planes).  Asynchronous on `stream`.
 */
int bf16_exp_decode(const uint8_t *d_in, uint64_t in_len, uint16_t *d_out, uint64_t n, uint32_t *d_status,
                    hipStream_t stream);

/* Static text for an ec_error value or for a set of EC_S_* status bits. */
const char *ec_error_string(int code);
const char *ec_status_string(uint32_t status);

#ifdef __cplusplus
}
#endif

#endif /* EC_H */
