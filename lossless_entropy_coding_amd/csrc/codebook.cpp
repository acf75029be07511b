// Host-side codebook construction for libec: ranking, Quad Length Codes,
// Huffman (two-queue merge + canonical codes) and Exp-Golomb on rank, plus
// the encode LUTs and the decode tables the GPU kernels read.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <numeric>
#include <vector>

#include "ec_internal.h"

namespace ec {
namespace {

uint64_t fnv1a64(const uint8_t *p, size_t n, uint64_t h = 0xcbf29ce484222325ull) {
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h;
}

// Symbols by decreasing count, equal counts by increasing byte value
// ("Quad Length Codes for Lossless Compression of e4m3", section 2: sorted
// by decreasing probability and indexed 0..255).
void rank_order(const uint64_t counts[256], uint8_t rank_to_sym[256]) {
    int order[256];
    std::iota(order, order + 256, 0);
    std::stable_sort(order, order + 256, [&](int a, int b) { return counts[a] > counts[b]; });
    for (int r = 0; r < 256; ++r) rank_to_sym[r] = (uint8_t)order[r];
}

ec_codebook *new_codebook(uint32_t codec) {
    ec_codebook *cb = new (std::nothrow) ec_codebook;
    if (!cb) return nullptr;
    memset(&cb->host, 0, sizeof(cb->host));
    memset(cb->area_size, 0, sizeof(cb->area_size));
    memset(cb->suffix_bits, 0, sizeof(cb->suffix_bits));
    cb->host.codec = codec;
    cb->host.eg_k = -1;
    return cb;
}

// Encode LUTs from per-symbol code values and lengths.
void fill_encode_luts(DevTables &t, const uint64_t code[256], const uint8_t len[256]) {
    uint32_t mx = 0;
    for (int s = 0; s < 256; ++s) {
        // code left-aligned (first code bit at bit 63 / 31), length in the low byte
        t.enc64[s] = (code[s] << (64 - len[s])) | len[s];
        t.code_len[s] = len[s];
        mx = std::max<uint32_t>(mx, len[s]);
    }
    t.max_len = mx;
    for (int s = 0; s < 256; ++s)
        t.enc32[s] = mx <= (uint32_t)kNarrowMaxLen ? ((uint32_t)code[s] << (32 - len[s])) | len[s] : 0u;
}

}  // namespace

// ------------------------------------------------------------------ QLC

int build_qlc(const uint64_t counts[256], const uint16_t area_size[8], const uint8_t suffix_bits[8],
              ec_codebook **out) {
    if (!counts || !area_size || !suffix_bits || !out) return EC_E_INVAL;
    uint32_t total = 0;
    for (int a = 0; a < 8; ++a) {
        if (suffix_bits[a] > 8 || area_size[a] > (1u << suffix_bits[a])) return EC_E_INVAL;
        total += area_size[a];
    }
    if (total != 256) return EC_E_INVAL;
    ec_codebook *cb = new_codebook(EC_CODEC_QLC);
    if (!cb) return EC_E_NOMEM;
    DevTables &t = cb->host;
    memcpy(cb->area_size, area_size, sizeof(cb->area_size));
    memcpy(cb->suffix_bits, suffix_bits, sizeof(cb->suffix_bits));
    rank_order(counts, t.sym);

    // area a covers ranks [first[a], first[a] + area_size[a]) and codes them
    // as the 3-bit prefix a followed by suffix_bits[a] offset bits
    uint32_t first[8];
    uint64_t code[256];
    uint8_t len[256];
    uint32_t r = 0;
    t.qlc_lens = 0;
    for (int a = 0; a < 8; ++a) {
        first[a] = r;
        t.qlc_lens |= (uint32_t)(3 + suffix_bits[a]) << (4 * a);
        for (uint32_t off = 0; off < area_size[a]; ++off, ++r) {
            uint8_t s = t.sym[r];
            code[s] = ((uint64_t)a << suffix_bits[a]) | off;
            len[s] = (uint8_t)(3 + suffix_bits[a]);
        }
    }
    fill_encode_luts(t, code, len);

    // level-1 decode: any 11-bit window starts with exactly one prefix; its
    // suffix is a codeword only below the area's symbol count
    for (uint32_t w = 0; w < (uint32_t)kL1Size; ++w) {
        uint32_t a = w >> 8;
        uint32_t b = suffix_bits[a];
        uint32_t s = b ? (w >> (8 - b)) & ((1u << b) - 1) : 0;
        t.l1[w] = s < area_size[a] ? t.sym[first[a] + s] : kQlcInvalid;
    }

    uint8_t desc[1 + 8 * 3 + 256];
    size_t k = 0;
    desc[k++] = EC_CODEC_QLC;
    for (int a = 0; a < 8; ++a) {
        desc[k++] = (uint8_t)(area_size[a] & 0xff);
        desc[k++] = (uint8_t)(area_size[a] >> 8);
        desc[k++] = suffix_bits[a];
    }
    memcpy(desc + k, t.sym, 256);
    k += 256;
    t.codebook_id = fnv1a64(desc, k);
    *out = cb;
    return EC_OK;
}

// QLC area layout with the fewest payload bits for these counts (QLC page,
// section 2: sizes and lengths of the areas adapt to the distribution, at
// most four distinct lengths; section 5: an optimised choice of both is the
// authors' next step).  With ranks sorted by decreasing count, some optimum
// has non-decreasing suffix widths, every non-empty area but the last full
// (2^width symbols) and the unused areas (size 0, width 0) at the end, so a
// layout is a non-decreasing width sequence that stops once its capacity
// reaches 256.  Dynamic programme over (first uncoded rank, areas used, last
// width, distinct widths): best[] holds the fewest bits for the ranks still
// to code; the layout is then read forwards taking the smallest width that
// keeps the optimum, which gives the lexicographically smallest width
// sequence among the cheapest layouts.
int qlc_optimal_areas(const uint64_t counts[256], uint32_t max_lengths, uint16_t area_size[8],
                      uint8_t suffix_bits[8]) {
    if (!counts || !area_size || !suffix_bits || max_lengths < 1 || max_lengths > 8) return EC_E_INVAL;
    typedef unsigned __int128 u128;
    const u128 kInf = ~(u128)0;
    uint8_t sym[256];
    rank_order(counts, sym);
    u128 P[257];   // P[i]: counts of ranks below i
    P[0] = 0;
    for (int r = 0; r < 256; ++r) P[r + 1] = P[r] + counts[sym[r]];

    // state (i, k, bp, d): ranks [i, 256) left, k areas used, last width bp,
    // d distinct widths so far
    static thread_local u128 best[257][9][9][9];
    static thread_local uint8_t seen[257][9][9][9];
    memset(seen, 0, sizeof(seen));
    // cost of the next area of width b at state (i, k, bp, d), kInf if not allowed
    auto step = [&](auto &self, uint32_t i, uint32_t k, uint32_t bp, uint32_t d, uint32_t b) -> u128 {
        const uint32_t nd = d + ((k == 0 || b != bp) ? 1u : 0u);
        if (nd > max_lengths) return kInf;
        const uint32_t n = std::min<uint32_t>(1u << b, 256 - i);
        const u128 c = (u128)(3 + b) * (P[i + n] - P[i]);
        if (i + n == 256) return c;
        if (k + 1 >= 8) return kInf;
        const u128 rest = self(self, i + n, k + 1, b, nd);
        return rest == kInf ? kInf : c + rest;
    };
    auto solve = [&](auto &self, uint32_t i, uint32_t k, uint32_t bp, uint32_t d) -> u128 {
        if (seen[i][k][bp][d]) return best[i][k][bp][d];
        u128 m = kInf;
        for (uint32_t b = (k ? bp : 0); b <= 8; ++b) m = std::min(m, step(self, i, k, bp, d, b));
        seen[i][k][bp][d] = 1;
        best[i][k][bp][d] = m;
        return m;
    };
    if (solve(solve, 0, 0, 0, 0) == kInf) return EC_E_INVAL;   // cannot happen: eight areas of 32 always fit

    uint32_t i = 0, k = 0, bp = 0, d = 0;
    for (int a = 0; a < 8; ++a) {
        area_size[a] = 0;
        suffix_bits[a] = 0;
    }
    while (i < 256) {
        const u128 target = best[i][k][bp][d];
        uint32_t b = k ? bp : 0;
        while (step(solve, i, k, bp, d, b) != target) ++b;
        const uint32_t n = std::min<uint32_t>(1u << b, 256 - i);
        area_size[k] = (uint16_t)n;
        suffix_bits[k] = (uint8_t)b;
        d += (k == 0 || b != bp) ? 1u : 0u;
        bp = b;
        i += n;
        ++k;
    }
    return EC_OK;
}

// -------------------------------------------------------------- Huffman

// Two-queue Huffman: leaves sorted by (weight, index) in one queue, merged
// nodes appended in creation order (their weights never decrease) to a
// second; each step takes the lighter front, a leaf on a tie.  This is the
// merge order of the key (weight, leaf before internal, index).
int huffman_lengths(const uint64_t *w, uint32_t n, uint8_t *len_out) {
    if (!w || !len_out || n < 2 || n > 256) return EC_E_INVAL;
    for (uint32_t i = 0; i < n; ++i)
        if (w[i] == 0) return EC_E_INVAL;
    std::vector<uint32_t> leaves(n);
    std::iota(leaves.begin(), leaves.end(), 0u);
    std::stable_sort(leaves.begin(), leaves.end(), [&](uint32_t a, uint32_t b) { return w[a] < w[b]; });
    std::vector<uint64_t> weight(2 * n);
    std::vector<uint32_t> parent(2 * n, 0);
    for (uint32_t i = 0; i < n; ++i) weight[i] = w[i];
    uint32_t li = 0;            // next leaf in sorted order
    uint32_t qh = n, qt = n;    // merged-node queue [qh, qt)
    auto take = [&]() -> uint32_t {
        if (li < n && (qh == qt || weight[leaves[li]] <= weight[qh])) return leaves[li++];
        return qh++;
    };
    for (uint32_t k = 0; k + 1 < n; ++k) {
        uint32_t a = take();
        uint32_t b = take();
        weight[qt] = weight[a] + weight[b];
        parent[a] = parent[b] = qt;
        ++qt;
    }
    // depths: the root is the last merged node; parents are created after
    // their children, so walk merged nodes from last to first
    std::vector<uint32_t> depth(2 * n, 0);
    const uint32_t root = qt - 1;
    for (uint32_t v = root; v-- > n;) depth[v] = depth[parent[v]] + 1;
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t d = depth[parent[i]] + 1;
        if (d > 255) return EC_E_UNSUPPORTED;
        len_out[i] = (uint8_t)d;
    }
    return EC_OK;
}

// Canonical codes from lengths (count per length, first code per length,
// codes handed out in increasing byte order within a length), then the
// encode LUTs and the two-level decode tables.
int build_huffman_lengths(const uint8_t len[256], ec_codebook **out) {
    if (!len || !out) return EC_E_INVAL;
    uint32_t bl_count[64] = {0};
    uint32_t mx = 0;
    for (int s = 0; s < 256; ++s) {
        if (len[s] == 0 || len[s] > EC_MAX_CODE_LEN) return len[s] ? EC_E_UNSUPPORTED : EC_E_INVAL;
        bl_count[len[s]]++;
        mx = std::max<uint32_t>(mx, len[s]);
    }
    // Kraft sum must be exactly 1 (a complete code): sum count[l] * 2^(mx-l) == 2^mx
    uint64_t kraft = 0;
    for (uint32_t l = 1; l <= mx; ++l) kraft += (uint64_t)bl_count[l] << (mx - l);
    if (kraft != (1ull << mx)) return EC_E_INVAL;

    ec_codebook *cb = new_codebook(EC_CODEC_HUFFMAN);
    if (!cb) return EC_E_NOMEM;
    DevTables &t = cb->host;
    // first code of length l = (first code of length l-1 + count of l-1) << 1
    uint64_t next_code[64] = {0};
    uint64_t c = 0;
    uint32_t idx = 0;
    for (uint32_t l = 1; l <= (uint32_t)EC_MAX_CODE_LEN; ++l) {
        c = (c + bl_count[l - 1]) << 1;      // bl_count[0] == 0
        next_code[l] = c;
        t.first_code[l] = c;
        t.first_idx[l] = idx;
        idx += bl_count[l];
    }
    uint64_t code[256];
    uint32_t fill[64];
    for (uint32_t l = 0; l < 64; ++l) fill[l] = 0;
    for (int s = 0; s < 256; ++s) {
        uint32_t l = len[s];
        code[s] = next_code[l]++;
        t.sym[t.first_idx[l] + fill[l]++] = (uint8_t)s;
    }
    fill_encode_luts(t, code, len);
    // 40-bit left-justified exclusive upper end of the codes of each length
    for (uint32_t l = 1; l <= (uint32_t)EC_MAX_CODE_LEN; ++l)
        t.limit[l] = ((uint64_t)t.first_code[l] + bl_count[l]) << (EC_MAX_CODE_LEN - l);

    // 13-bit decode table: windows whose code has <= 13 bits hold its length
    // in the low byte and its byte value in the high byte (a shift by the
    // entry then moves past the code); 0 marks the prefixes of longer codes
    // (found by the canonical limit search)
    for (int w = 0; w < kHuffSize; ++w) t.hl1[w] = 0;
    for (int s = 0; s < 256; ++s) {
        uint32_t l = len[s];
        if (l == 0 || l > (uint32_t)kHuffBits) continue;
        uint32_t lo = (uint32_t)code[s] << (kHuffBits - l), hi = lo + (1u << (kHuffBits - l));
        for (uint32_t w = lo; w < hi; ++w) t.hl1[w] = (uint16_t)(l | ((uint32_t)s << 8));
    }

    uint8_t desc[257];
    desc[0] = EC_CODEC_HUFFMAN;
    memcpy(desc + 1, len, 256);
    t.codebook_id = fnv1a64(desc, 257);
    *out = cb;
    return EC_OK;
}

// ------------------------------------------------------------ Exp-Golomb

namespace {
// order-k Exp-Golomb length of a rank: 2 * floor(log2(rank + 2^k)) - k + 1
uint32_t eg_len(uint32_t rank, uint32_t k) {
    uint32_t v = rank + (1u << k);
    uint32_t m = 31 - (uint32_t)__builtin_clz(v);
    return 2 * m - k + 1;
}
}  // namespace

int build_eg(const uint64_t counts[256], int k, ec_codebook **out) {
    if (!counts || !out || k < -1 || k > 8) return EC_E_INVAL;
    ec_codebook *cb = new_codebook(EC_CODEC_EXP_GOLOMB);
    if (!cb) return EC_E_NOMEM;
    DevTables &t = cb->host;
    rank_order(counts, t.sym);
    if (k < 0) {
        unsigned __int128 best = 0;
        for (uint32_t kk = 0; kk <= 8; ++kk) {
            unsigned __int128 bits = 0;
            for (uint32_t r = 0; r < 256; ++r) bits += (unsigned __int128)counts[t.sym[r]] * eg_len(r, kk);
            if (kk == 0 || bits < best) {
                best = bits;
                k = (int)kk;
            }
        }
    }
    t.eg_k = k;
    uint64_t code[256];
    uint8_t len[256];
    for (uint32_t r = 0; r < 256; ++r) {
        uint8_t s = t.sym[r];
        code[s] = r + (1u << k);      // the m - k leading zeros are implicit in the length
        len[s] = (uint8_t)eg_len(r, (uint32_t)k);
    }
    fill_encode_luts(t, code, len);
    uint8_t desc[2 + 256];
    desc[0] = EC_CODEC_EXP_GOLOMB;
    desc[1] = (uint8_t)k;
    memcpy(desc + 2, t.sym, 256);
    t.codebook_id = fnv1a64(desc, sizeof(desc));
    *out = cb;
    return EC_OK;
}

}  // namespace ec
