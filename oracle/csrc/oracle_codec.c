/*
 * Plain, scalar, single-threaded CPU oracle for the e4m3 entropy codecs.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link or call
 * this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or table with the GPU library.
 *
 * Everything here is bit-serial on purpose: one call of put_bit / get_bit per
 * coded bit, so that a reader can check each step against the definitions.
 *
 * Bit order of the payload (the container is this project's own; the pages
 * define codes, not a byte format): the payload of a chunk is a sequence of
 * 32-bit little-endian words, and stream bit i of the chunk is bit
 * (31 - i % 32) of word i / 32.  Codes are written most significant bit
 * first, in symbol order.  Bits after the last code, up to the chunk's
 * 16-byte boundary, are zero.
 */
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- histogram */

/* counts[s] = number of positions i with x[i] == s. */
void orc_histogram(const uint8_t *x, uint64_t n, uint64_t *counts)
{
    for (int s = 0; s < 256; s++)
        counts[s] = 0;
    for (uint64_t i = 0; i < n; i++)
        counts[x[i]] += 1;
}

/* ------------------------------------------------------------------ bit I/O */

static void put_bit(uint8_t *chunk, uint64_t pos, int bit)
{
    uint64_t word = pos / 32;
    int k = 31 - (int)(pos % 32);            /* bit index inside the word */
    uint64_t byte = word * 4 + (uint64_t)(k / 8); /* little-endian word */
    if (bit)
        chunk[byte] |= (uint8_t)(1u << (k % 8));
}

static int get_bit(const uint8_t *chunk, uint64_t pos)
{
    uint64_t word = pos / 32;
    int k = 31 - (int)(pos % 32);
    uint64_t byte = word * 4 + (uint64_t)(k / 8);
    return (chunk[byte] >> (k % 8)) & 1;
}

/* ------------------------------------------------------------------ encoder */

/*
 * Encode x[0..n) chunk by chunk with a fixed per-symbol code table:
 * symbol s is written as the len[s] low bits of code[s], MSB first.
 *
 *   chunk_symbols  C, a multiple of 256
 *   payload        zero-initialised by this function, payload_cap bytes
 *   chunk_off      [n_chunks + 1] byte offsets of each chunk in the payload
 *   sub_end        [n_chunks][C / 256] bit offset, from the chunk start, of the
 *                  end of each 256-symbol sub-chunk; sub-chunks that lie past
 *                  n hold the chunk's total bit count
 *
 * Returns the payload size in bytes, or UINT64_MAX if payload_cap is too small.
 */
uint64_t orc_encode(const uint8_t *x, uint64_t n, uint32_t chunk_symbols,
                    const uint64_t *code, const uint8_t *len,
                    uint8_t *payload, uint64_t payload_cap,
                    uint64_t *chunk_off, uint32_t *sub_end)
{
    const uint64_t C = chunk_symbols;
    const uint64_t subs = C / 256;
    const uint64_t n_chunks = (n + C - 1) / C;
    memset(payload, 0, payload_cap);

    uint64_t off = 0;
    chunk_off[0] = 0;
    for (uint64_t c = 0; c < n_chunks; c++) {
        uint64_t first = c * C;
        uint64_t last = first + C < n ? first + C : n;
        uint64_t bits = 0;
        for (uint64_t i = first; i < last; i++) {
            uint8_t s = x[i];
            int l = len[s];
            if (off + (bits + (uint64_t)l + 7) / 8 > payload_cap)
                return UINT64_MAX;
            for (int b = l - 1; b >= 0; b--) {
                put_bit(payload + off, bits, (int)((code[s] >> b) & 1));
                bits += 1;
            }
            uint64_t done = i + 1 - first;
            if (done % 256 == 0)
                sub_end[c * subs + done / 256 - 1] = (uint32_t)bits;
        }
        /* the unfinished sub-chunk and those past n end where the chunk ends */
        uint64_t done = last - first;
        for (uint64_t j = done / 256; j < subs; j++)
            sub_end[c * subs + j] = (uint32_t)bits;
        uint64_t bytes = (bits + 7) / 8;
        bytes = (bytes + 15) / 16 * 16;
        off += bytes;
        chunk_off[c + 1] = off;
    }
    return off;
}

/* ---------------------------------------------------------------- decoders */

/* common checks after a sub-chunk: the read position must be its recorded end */
static int sub_ok(uint64_t pos, const uint32_t *sub_end, uint64_t c, uint64_t subs, uint64_t j)
{
    return pos == sub_end[c * subs + j];
}

/* the bits between the last code and the chunk's padded end must be zero */
static int padding_ok(const uint8_t *chunk, uint64_t pos, uint64_t chunk_bytes)
{
    for (uint64_t p = pos; p < chunk_bytes * 8; p++)
        if (get_bit(chunk, p))
            return 0;
    return 1;
}

/* Return codes shared by the decoders. */
enum { ORC_OK = 0, ORC_CORRUPT = 1 };

/*
 * QLC decoder: read the 3-bit area prefix, which fixes the code length; read
 * that area's suffix bits; the rank is the area's first rank plus the suffix;
 * a second table maps the rank back to the byte.  A suffix at or beyond the
 * area's symbol count is not a codeword.
 */
int orc_decode_qlc(const uint8_t *payload, uint64_t payload_bytes,
                   const uint64_t *chunk_off, const uint32_t *sub_end,
                   uint64_t n, uint32_t chunk_symbols,
                   const uint16_t *area_size, const uint8_t *suffix_bits,
                   const uint8_t *rank_to_sym, uint8_t *out)
{
    const uint64_t C = chunk_symbols, subs = C / 256;
    const uint64_t n_chunks = (n + C - 1) / C;
    uint32_t area_first[8];
    uint32_t acc = 0;
    for (int a = 0; a < 8; a++) {
        area_first[a] = acc;
        acc += area_size[a];
    }
    for (uint64_t c = 0; c < n_chunks; c++) {
        if (chunk_off[c + 1] > payload_bytes || chunk_off[c] > chunk_off[c + 1])
            return ORC_CORRUPT;
        const uint8_t *chunk = payload + chunk_off[c];
        uint64_t chunk_bits = (chunk_off[c + 1] - chunk_off[c]) * 8;
        uint64_t first = c * C, last = first + C < n ? first + C : n;
        uint64_t pos = 0;
        for (uint64_t i = first; i < last; i++) {
            if (pos + 3 > chunk_bits)
                return ORC_CORRUPT;
            int area = 0;
            for (int b = 0; b < 3; b++)
                area = area * 2 + get_bit(chunk, pos++);
            int w = suffix_bits[area];
            if (pos + (uint64_t)w > chunk_bits)
                return ORC_CORRUPT;
            uint32_t suffix = 0;
            for (int b = 0; b < w; b++)
                suffix = suffix * 2 + (uint32_t)get_bit(chunk, pos++);
            if (suffix >= area_size[area])
                return ORC_CORRUPT;
            out[i] = rank_to_sym[area_first[area] + suffix];
            uint64_t done = i + 1 - first;
            if (done % 256 == 0 && !sub_ok(pos, sub_end, c, subs, done / 256 - 1))
                return ORC_CORRUPT;
        }
        if ((last - first) % 256 && !sub_ok(pos, sub_end, c, subs, (last - first) / 256))
            return ORC_CORRUPT;
        if (!padding_ok(chunk, pos, chunk_off[c + 1] - chunk_off[c]))
            return ORC_CORRUPT;
    }
    return ORC_OK;
}

/*
 * Huffman decoder: walk the code tree one bit at a time from the root.
 * child[2 * node + bit] is the next node; a value < 0 is a leaf holding
 * symbol -(value + 1).  Node 0 is the root.
 */
int orc_decode_huffman(const uint8_t *payload, uint64_t payload_bytes,
                       const uint64_t *chunk_off, const uint32_t *sub_end,
                       uint64_t n, uint32_t chunk_symbols,
                       const int32_t *child, uint8_t *out)
{
    const uint64_t C = chunk_symbols, subs = C / 256;
    const uint64_t n_chunks = (n + C - 1) / C;
    for (uint64_t c = 0; c < n_chunks; c++) {
        if (chunk_off[c + 1] > payload_bytes || chunk_off[c] > chunk_off[c + 1])
            return ORC_CORRUPT;
        const uint8_t *chunk = payload + chunk_off[c];
        uint64_t chunk_bits = (chunk_off[c + 1] - chunk_off[c]) * 8;
        uint64_t first = c * C, last = first + C < n ? first + C : n;
        uint64_t pos = 0;
        for (uint64_t i = first; i < last; i++) {
            int32_t node = 0;
            for (;;) {
                if (pos >= chunk_bits)
                    return ORC_CORRUPT;
                int32_t next = child[2 * node + get_bit(chunk, pos++)];
                if (next < 0) {
                    out[i] = (uint8_t)(-(next + 1));
                    break;
                }
                if (next == 0)          /* unused branch of an incomplete tree */
                    return ORC_CORRUPT;
                node = next;
            }
            uint64_t done = i + 1 - first;
            if (done % 256 == 0 && !sub_ok(pos, sub_end, c, subs, done / 256 - 1))
                return ORC_CORRUPT;
        }
        if ((last - first) % 256 && !sub_ok(pos, sub_end, c, subs, (last - first) / 256))
            return ORC_CORRUPT;
        if (!padding_ok(chunk, pos, chunk_off[c + 1] - chunk_off[c]))
            return ORC_CORRUPT;
    }
    return ORC_OK;
}

/*
 * Order-k Exp-Golomb decoder: count leading zeros z one bit at a time, then
 * read z + k + 1 bits (the first is the 1 that stopped the count) as v; the
 * rank is v - 2^k.  Ranks above 255 are not codewords.
 */
int orc_decode_eg(const uint8_t *payload, uint64_t payload_bytes,
                  const uint64_t *chunk_off, const uint32_t *sub_end,
                  uint64_t n, uint32_t chunk_symbols,
                  uint32_t k, const uint8_t *rank_to_sym, uint8_t *out)
{
    const uint64_t C = chunk_symbols, subs = C / 256;
    const uint64_t n_chunks = (n + C - 1) / C;
    for (uint64_t c = 0; c < n_chunks; c++) {
        if (chunk_off[c + 1] > payload_bytes || chunk_off[c] > chunk_off[c + 1])
            return ORC_CORRUPT;
        const uint8_t *chunk = payload + chunk_off[c];
        uint64_t chunk_bits = (chunk_off[c + 1] - chunk_off[c]) * 8;
        uint64_t first = c * C, last = first + C < n ? first + C : n;
        uint64_t pos = 0;
        for (uint64_t i = first; i < last; i++) {
            uint32_t z = 0;
            for (;;) {
                if (pos >= chunk_bits || z > 16)
                    return ORC_CORRUPT;
                if (get_bit(chunk, pos))
                    break;
                z++;
                pos++;
            }
            uint64_t v = 0;
            for (uint32_t b = 0; b < z + k + 1; b++) {
                if (pos >= chunk_bits)
                    return ORC_CORRUPT;
                v = v * 2 + (uint64_t)get_bit(chunk, pos++);
            }
            uint64_t rank = v - ((uint64_t)1 << k);
            if (rank > 255)
                return ORC_CORRUPT;
            out[i] = rank_to_sym[rank];
            uint64_t done = i + 1 - first;
            if (done % 256 == 0 && !sub_ok(pos, sub_end, c, subs, done / 256 - 1))
                return ORC_CORRUPT;
        }
        if ((last - first) % 256 && !sub_ok(pos, sub_end, c, subs, (last - first) / 256))
            return ORC_CORRUPT;
        if (!padding_ok(chunk, pos, chunk_off[c + 1] - chunk_off[c]))
            return ORC_CORRUPT;
    }
    return ORC_OK;
}
