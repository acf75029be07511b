// Chunk-parallel decoder.
//
// Every 256-symbol sub-chunk starts at a bit offset recorded in the stream
// index, so one lane decodes one sub-chunk serially and a wave64 decodes 64
// consecutive sub-chunks side by side (a "run").  Each lane's serial chain is
// bound by LDS latency (about 70 cycles a table or window read), so the
// decoder keeps as many chains in flight as a CU holds: sixteen waves, one
// workgroup per CU, which covers a 64 MiB shard (4096 runs) in one round.
//
// LDS ring.  A lane's bits reach LDS through a ring of eight 16-byte blocks
// in its own column of the wave's region: word k of the lane's data sits in
// row (k + 1) mod 32, one 4-byte column per lane, so a 32-bit window at any
// bit position is one read of two rows plus a funnel shift, and the 64 lanes
// of a read always hit 64 different banks.  Rows 32 and 33 repeat rows 0 and
// 1, so a window that reaches past row 31 reads on without wrapping.  A run
// starts with its ring full, eight blocks a lane loaded by lane quads (four
// lanes read 64 consecutive bytes of one lane's sub-chunk per load and write
// them into that lane's column).  Two register buffers of two blocks then
// take turns at uniform refill points every 16 symbols: a lane writes the
// turn's buffer into its ring if it holds blocks, then reloads it with its
// next two blocks not already in the other buffer when the ring will have
// room for them two points later (else it loads one block that all such
// lanes share: one request).  So a buffer's blocks are always written at its
// next turn, two points (32 symbols) after their loads were issued, and
// every point issues the same two load instructions: the wave waits for the
// loads of two points before, never for the ones just issued, and no block
// is requested twice.  Ring addresses are taken modulo the ring, so no read ever
// leaves the region, whatever the data.  A lane that consumed bits the ring did not
// yet hold (more than 16 bits a symbol for 32 symbols: long codes only)
// decodes its run again from global memory afterwards.
//   QLC      the 3-bit prefix gives the code length through a funnel shift
//            and a byte permute of the per-area lengths (no memory access on
//            the dependency chain); the top 11 bits index a 2048-entry LDS
//            table that yields the byte or flags an unused suffix.
//   Huffman  the top 13 bits index a 16 KiB LDS table that yields the length
//            (low byte: a shift by the entry itself moves past the code) and
//            the byte (high byte) of every code of up to 13 bits; longer codes
//            (rare) are found by comparing a 40-bit window against the
//            canonical code limits.
//   EG       count leading zeros z; the code is 2z + k + 1 bits; rank -> byte
//            through a 256-entry LDS table.
// Decoded bytes gather in registers, 64 bytes per lane, and leave as whole
// 64-byte pieces after a turn-around among four lanes, one 16-byte streaming
// store per refill point (so that a store is never among the memory
// operations a refill waits for; see the kernel).  The ring path serves waves
// whose 64 lanes all hold whole sub-chunks; a wave with a shorter or missing
// sub-chunk (a segment's last run) or an index found corrupt decodes straight
// from global memory instead.  After its last symbol a lane checks that it
// stopped exactly where the index says its sub-chunk ends, and the lane of a
// chunk's last sub-chunk checks that the padding after it is zero.
#include "dev_common.h"

namespace ec {

namespace {

// Waves of the one workgroup per CU: sixteen (128 registers each) for QLC
// and Huffman; eight for Exp-Golomb, whose parse needs about 200 registers.
template <int CODEC>
constexpr int waves_for() {
    return CODEC == EC_CODEC_EXP_GOLOMB ? 8 : 16;
}
constexpr uint32_t kLdsBytes = 160 * 1024;
constexpr uint32_t kRowBytes = 64 * 4;             // one word per lane
constexpr uint32_t kRingBlocks = 8;                // 16-byte blocks a lane holds in LDS
constexpr uint32_t kRingRows = 4 * kRingBlocks;    // 32 word rows
constexpr uint32_t kRegionRows = kRingRows + 2;    // plus copies of rows 0 and 1
constexpr uint32_t kBatch = 2;                     // blocks per refill buffer
constexpr uint32_t kNone = 0xffffffffu;            // refill buffer holding no blocks of the lane

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) const uint32_t lds_word;

// Bits of a lane's run read from its ring.  Y is the lane-relative bit
// position plus 31: the row holding the bit before the position is
// (Y >> 5) mod 32 (word k sits in row k + 1), and a window at a word boundary
// reads that row and shifts it out.
struct RingBits {
    uint32_t Y;
    uint32_t rbase;   // LDS byte address of the lane's column in row 0

    __device__ __forceinline__ lds_word *row(uint32_t yy) const {
        return (lds_word *)(size_t)(rbase + (((yy >> 5) & (kRingRows - 1)) << 8));
    }
    __device__ __forceinline__ uint32_t win() const {
        lds_word *w = row(Y);
        return __builtin_amdgcn_alignbit(w[0], w[64], ~Y);
    }
    __device__ __forceinline__ uint64_t win64() const {   // rows k, k + 1, k + 2 of the column
        lds_word *w = row(Y);
        const uint32_t d0 = w[0], d1 = w[64], d2 = w[128];
        return ((uint64_t)__builtin_amdgcn_alignbit(d0, d1, ~Y) << 32) | __builtin_amdgcn_alignbit(d1, d2, ~Y);
    }
    __device__ __forceinline__ void adv(uint32_t l) { Y += l; }
    __device__ __forceinline__ void prepare() {}
    __device__ __forceinline__ uint32_t bit() const { return Y - 31; }
};

// Bits of a lane's sub-chunk read straight from global memory (runs the ring
// did not serve): a 64-bit MSB-aligned buffer refilled 32 bits at a time,
// loads clamped to the payload.
struct GlobalBits {
    const uint32_t *base;   // lane's first payload word
    uint32_t last;          // last readable word, relative to base (clamped)
    uint64_t buf;           // next stream bits, MSB-aligned
    uint32_t nb;            // valid bits in buf (>= 32 between calls)
    uint32_t nxt;           // next word to fetch, relative to base
    uint64_t base0;         // absolute index of base

    __device__ __forceinline__ uint32_t word(uint32_t i) const { return base[i < last ? i : last]; }
    __device__ __forceinline__ void init(const uint32_t *payload, uint64_t n_words, uint64_t bitpos) {
        const uint64_t w0 = bitpos >> 5;
        const uint64_t lastw = n_words - 1;
        const uint64_t b = w0 < lastw ? w0 : lastw;
        base = payload + b;
        // a run never reads more than a few hundred words past its start
        last = (uint32_t)min(lastw - b, (uint64_t)0xffffffffu);
        base0 = w0;
        const uint32_t o = (uint32_t)(bitpos & 31);
        buf = (((uint64_t)word(0) << 32) | word(1)) << o;
        nb = 64 - o;
        nxt = 2;
        fill();
    }
    __device__ __forceinline__ void fill() {
        while (nb <= 32) {
            buf |= (uint64_t)word(nxt) << (32 - nb);
            nb += 32;
            ++nxt;
        }
    }
    __device__ __forceinline__ uint32_t win() const { return (uint32_t)(buf >> 32); }
    __device__ __forceinline__ uint64_t win64() const {
        return buf | (nb <= 32 ? (uint64_t)word(nxt) << (32 - nb) : (uint64_t)word(nxt) >> (nb - 32));
    }
    __device__ __forceinline__ void adv(uint32_t l) {
        if (l >= nb) {   // codes longer than the buffered bits (deep Huffman codes)
            l -= nb;
            buf = 0;
            nb = 0;
            fill();
        }
        buf <<= l;
        nb -= l;
        fill();
    }
    __device__ __forceinline__ void prepare() {}
    __device__ __forceinline__ uint64_t bit() const { return (base0 + nxt) * 32 - nb; }
};

// Canonical-code tables for Huffman codes longer than the decode table's 13
// bits, copied to LDS (lengths 14..40).
struct DeepTables {
    uint64_t limit[EC_MAX_CODE_LEN - kHuffBits];        // 40-bit left-justified end of the codes of length l
    uint64_t first_code[EC_MAX_CODE_LEN - kHuffBits];   // canonical first code of length l
    uint32_t first_idx[EC_MAX_CODE_LEN - kHuffBits];    // its position in the canonical symbol order
};

// Huffman code longer than 13 bits (rare): canonical limit search on a
// 40-bit left-justified window.  Returns length | symbol << 8, the format
// of the decode table's entries.  Inlined: a called function starts by
// waiting for every memory operation in flight, which would drain the
// decoder's refill loads each time a wave meets a long code.
__device__ __forceinline__ uint32_t huff_deep(uint64_t window, const DeepTables *dt, const uint8_t *sym, uint32_t mx) {
    const uint64_t w40 = window >> (64 - EC_MAX_CODE_LEN);
    uint32_t l = kHuffBits + 1;
    while (l < mx && w40 >= dt->limit[l - kHuffBits - 1]) ++l;
    const uint32_t i = l - kHuffBits - 1;
    const uint64_t code = w40 >> (EC_MAX_CODE_LEN - l);
    const uint32_t idx = dt->first_idx[i] + (uint32_t)(code - dt->first_code[i]);
    return l | ((uint32_t)sym[idx & 255] << 8);
}

// Status bits from a rare path, behind a call: the decode loop then has a
// fixed number of memory operations, and the compiler counts the loads in
// flight exactly instead of waiting for every store.
__device__ __noinline__ void flag(uint32_t *status, uint32_t bits) { or_status(status, bits); }

// Whether any bit of the payload in [from, to) is set: the zero padding
// between a chunk's last code and its end (to is a multiple of 32, since
// chunks start at 16-byte offsets).  Behind a call, like every rare path.
__device__ __noinline__ bool padding_set(const uint32_t *payload, uint64_t from, uint64_t to) {
    uint32_t any = 0;
    for (uint64_t w = from >> 5; w < (to >> 5); ++w) {
        uint32_t x = payload[w];
        if (w == (from >> 5)) x &= 0xffffffffu >> (from & 31);   // bits at and after `from` (MSB first)
        any |= x;
    }
    return any != 0;
}

// Code parsing over a bit source S.  bad collects the QLC / EG "not a
// codeword" flags (bit 8 and up).
template <int CODEC, int PAIRS, class Src>
struct Codes {
    Src &S;
    const void *tab;   // QLC: u32 entries; Huffman: u16 entries
    const uint8_t *symtab;
    const DeepTables *dt;
    uint32_t max_len, k_eg;
    uint32_t llo, lhi;   // QLC code lengths by area, one byte each: areas 0-3 in llo, 4-7 in lhi
    uint32_t bad;

    __device__ __forceinline__ Codes(Src &s, const void *tab_, const uint8_t *symtab_, const DeepTables *dt_,
                                     uint32_t max_len_, uint32_t lens, uint32_t k_eg_)
        : S(s), tab(tab_), symtab(symtab_), dt(dt_), max_len(max_len_), k_eg(k_eg_), llo(0), lhi(0), bad(0) {
        if (CODEC == EC_CODEC_QLC) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                llo |= ((lens >> (4 * k)) & 15u) << (8 * k);
                lhi |= ((lens >> (4 * k + 16)) & 15u) << (8 * k);
            }
        }
    }

    // The code that starts window w: its table entry and its length.  QLC
    // and EG entries hold the symbol in byte 0 (QLC: bit 8 flags an unused
    // suffix); Huffman entries hold the length in byte 0 and the symbol in
    // byte 1 (0: a code longer than the table covers).  QLC takes the length
    // from the 3-bit prefix, off the memory dependency chain: a funnel shift
    // puts the prefix in byte 0 of a byte-select word whose other bytes
    // select zero, and a byte permute picks that area's length.
    struct Code {
        uint32_t e, len;
    };
    __device__ __forceinline__ const uint16_t *hl1() const { return static_cast<const uint16_t *>(tab); }
    __device__ __forceinline__ Code code_at(uint32_t w) {
        if (CODEC == EC_CODEC_QLC) {
            const uint32_t sel = __builtin_amdgcn_alignbit(0x01818180u, w, 29);   // 0x0c0c0c00 | w >> 29
            return Code{static_cast<const uint32_t *>(tab)[w >> 21], __builtin_amdgcn_perm(lhi, llo, sel)};
        } else if (CODEC == EC_CODEC_HUFFMAN) {
            uint32_t e = hl1()[w >> (32 - kHuffBits)];
            if (e == 0u) e = huff_deep(S.win64(), dt, symtab, max_len);
            return Code{e, e & 0xffu};
        } else {
            const uint32_t zr = __clz(w);
            const uint32_t z = zr < 8u ? zr : 8u;   // more zeros: not a codeword
            const uint32_t l = 2 * z + k_eg + 1;
            const uint32_t rank = (w >> (32 - l)) - (1u << k_eg);
            bad |= rank | (zr > 8u ? kQlcInvalid : 0u);
            return Code{symtab[rank & 255u], l};
        }
    }
    // the symbol of an entry, and the byte permute that takes the symbols of
    // two entries (first in byte 0, second in byte 1)
    static constexpr uint32_t kSymShift = CODEC == EC_CODEC_HUFFMAN ? 8 : 0;
    static constexpr uint32_t kPairSel = CODEC == EC_CODEC_HUFFMAN ? 0x0c0c0501u : 0x0c0c0400u;

    __device__ __forceinline__ uint32_t one() {
        const Code c = code_at(S.win());
        if (CODEC == EC_CODEC_QLC) bad |= c.e;
        S.adv(c.len);
        return (c.e >> kSymShift) & 0xffu;
    }
    // two codes from one window when both fit in it; returns byte0 | byte1 << 8
    __device__ __forceinline__ uint32_t two() {
        const uint32_t w = S.win();
        Code c1, c2;
        if (CODEC == EC_CODEC_HUFFMAN) {
            // Both table reads from the one window: a code the table covers
            // has at most 13 bits, so 19 bits of the window follow it.  A
            // longer code (rare) sends the lanes that hold one to the
            // canonical search and a fresh window for the second code.
            // (shifts take their amount modulo 32: a shift by the entry is
            // a shift by the code's length)
            uint32_t e1 = hl1()[w >> (32 - kHuffBits)];
            uint32_t e2 = hl1()[(w << (e1 & 31u)) >> (32 - kHuffBits)];
            if (min(e1, e2) == 0u) {
                if (e1 == 0u) e1 = huff_deep(S.win64(), dt, symtab, max_len);
                S.adv(e1 & 0xffu);
                e2 = hl1()[S.win() >> (32 - kHuffBits)];
                if (e2 == 0u) e2 = huff_deep(S.win64(), dt, symtab, max_len);
                S.adv(e2 & 0xffu);
            } else {
                S.adv((e1 + e2) & 0xffu);   // lengths of at most 13 bits: no carry into the symbols
            }
            c1.e = e1;
            c2.e = e2;
        } else {
            c1 = code_at(w);
            c2 = code_at(w << c1.len);
            S.adv(c1.len + c2.len);
            if (CODEC == EC_CODEC_QLC) bad |= c1.e | c2.e;
        }
        return __builtin_amdgcn_perm(c2.e, c1.e, kPairSel);   // c1's symbol, c2's symbol
    }
    // Four codes from one 64-bit window: the second pair's 32-bit window lies
    // inside the 64 bits when a pair has at most 32 bits (QLC: codes of at
    // most 11 bits; EG in pair mode: at most 16; Huffman: codes the table
    // covers, at most 13 bits each, else (rare) the pair step twice).
    // Returns the four bytes in order.
    __device__ __forceinline__ uint32_t four() {
        const uint64_t W = S.win64();
        const uint32_t w = (uint32_t)(W >> 32);
        if (CODEC != EC_CODEC_HUFFMAN) {
            const Code c1 = code_at(w);
            const Code c2 = code_at(w << c1.len);
            const uint32_t L1 = c1.len + c2.len;
            const uint32_t v = (uint32_t)((W << L1) >> 32);
            const Code c3 = code_at(v);
            const Code c4 = code_at(v << c3.len);
            S.adv(L1 + c3.len + c4.len);
            if (CODEC == EC_CODEC_QLC) bad |= c1.e | c2.e | c3.e | c4.e;
            return __builtin_amdgcn_perm(c2.e, c1.e, 0x0c0c0400u) | (__builtin_amdgcn_perm(c4.e, c3.e, 0x0c0c0400u) << 16);
        }
        // entries hold the length in their low byte: shifts by an entry (or
        // by the sum of two, for the 64-bit shift, modulo 64) move past the codes
        const uint32_t e1 = hl1()[w >> (32 - kHuffBits)];
        const uint32_t e2 = hl1()[(w << (e1 & 31u)) >> (32 - kHuffBits)];
        const uint32_t e12 = e1 + e2;   // lengths add in the low byte (at most 26)
        const uint32_t v = (uint32_t)((W << (e12 & 63u)) >> 32);
        const uint32_t e3 = hl1()[v >> (32 - kHuffBits)];
        const uint32_t e4 = hl1()[(v << (e3 & 31u)) >> (32 - kHuffBits)];
        if (min(min(e1, e2), min(e3, e4)) == 0u) {
            const uint32_t p0 = two(), p1 = two();
            return p0 | (p1 << 16);
        }
        S.adv((e12 + e3 + e4) & 0xffu);
        return __builtin_amdgcn_perm(e2, e1, kPairSel) | (__builtin_amdgcn_perm(e4, e3, kPairSel) << 16);
    }
    // eight codes -> two output words
    __device__ __forceinline__ void eight(uint32_t &lo, uint32_t &hi) {
        S.prepare();
        if (PAIRS) {
            lo = four();
            hi = four();
        } else {
            uint32_t b[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) b[k] = one();
            lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
            hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        }
    }
};

// A lane's sub-chunk: its bits [sb, eb) in the payload and its symbols,
// and the 16-byte payload blocks that hold them.
struct LaneTask {
    uint64_t sb, eb;
    uint64_t pad_end;   // the chunk's end bit when this is its last sub-chunk, else 0
    uint64_t first_sym;
    uint64_t blk0;      // first block
    uint32_t nv;        // blocks (0: nothing to decode)
    uint32_t cnt;       // symbols (0: no sub-chunk)
    bool ok;            // index entries valid
};

// Index entries of a lane's sub-chunk as loaded (resolved later, so that the
// loads are in flight while the wave decodes an earlier run).
struct IndexRaw {
    uint32_t co0, co1;        // the lane's chunk: offsets of its start and end in the payload, 16-byte units
    uint32_t e_start, e_end;  // the lane's sub-chunk: start and end bit in its chunk
    bool last;                // the sub-chunk is its chunk's last: the padding after it is checked
};

// Stream fields the runs of a segment share (validated once per segment).
struct StreamInfo {
    const uint8_t *stream;
    uint64_t po, pb;
    uint32_t nch, spc;
};

__device__ __forceinline__ IndexRaw issue_index(const DecodeArgs &a, const StreamInfo &si, uint32_t g) {
    const uint64_t *chunk_off = reinterpret_cast<const uint64_t *>(si.stream + kHeaderBytes);
    const uint32_t *sub_end = reinterpret_cast<const uint32_t *>(si.stream + kHeaderBytes + 8ull * (si.nch + 1));
    const uint32_t gl = g < a.blocks_per_seg ? g : a.blocks_per_seg - 1;
    const uint32_t c = gl / si.spc, j = gl - c * si.spc;
    IndexRaw r;
    // offsets are 16-byte aligned and below 2^36 (checked with the header):
    // kept as 32-bit counts of 16 bytes; a misaligned one reads as corrupt
    const uint64_t o0 = chunk_off[c], o1 = chunk_off[c + 1];
    r.co0 = (o0 & 15) || (o0 >> 36) ? 0xffffffffu : (uint32_t)(o0 >> 4);
    r.co1 = (o1 & 15) || (o1 >> 36) ? 0u : (uint32_t)(o1 >> 4);
    r.e_end = sub_end[(uint64_t)c * si.spc + j];
    // (loaded for every lane, so that the number of loads is fixed)
    const uint32_t prev = sub_end[(uint64_t)c * si.spc + j - (j ? 1u : 0u)];
    r.e_start = j ? prev : 0u;
    r.last = j == si.spc - 1 || gl == a.blocks_per_seg - 1;
    return r;
}

// Checks the index entries of sub-chunk g (flags a corrupt index).
__device__ __forceinline__ LaneTask resolve(const DecodeArgs &a, const StreamInfo &si, const IndexRaw &r, uint32_t g,
                                            uint32_t *status) {
    const bool active = g < a.blocks_per_seg;
    LaneTask t;
    const uint64_t co0 = (uint64_t)r.co0 * 16, co1 = (uint64_t)r.co1 * 16;
    t.ok = active && r.co0 <= r.co1 && co1 <= si.pb && (uint64_t)r.e_end <= (co1 - co0) * 8 && r.e_start <= r.e_end;
    if (active && !t.ok) flag(status, EC_S_CORRUPT);
    t.sb = co0 * 8 + r.e_start;
    t.eb = co0 * 8 + r.e_end;
    t.pad_end = r.last ? co1 * 8 : 0;
    t.first_sym = (uint64_t)g * kSub;
    t.cnt = !active ? 0u : (a.seg_n - t.first_sym < kSub ? (uint32_t)(a.seg_n - t.first_sym) : (uint32_t)kSub);
    const bool live = t.ok && t.cnt > 0 && t.eb > t.sb;
    t.blk0 = live ? t.sb >> 7 : 0;
    t.nv = live ? (uint32_t)(((t.eb - 1) >> 7) - t.blk0 + 1) : 0u;
    return t;
}

// A run's first eight blocks per lane, the whole ring, loaded by lane quads:
// in load 2 k + h, lane 4 j + p takes block 4 h + p of lane 4 j + k's
// sub-chunk, so the quad reads 64 consecutive bytes (one or two line requests
// where four lanes on their own lines make four).  Fewer requests shorten the
// fills of later runs, which queue behind other waves' refills and stores;
// the very first fills of a launch, every wave of the chip asking at once,
// are bound by the bytes either way.  Block indexes are clamped to the
// owner's last block (every lane of a ring run holds at least one), so every
// load stays inside the payload.
__device__ __forceinline__ void issue_fill(const StreamInfo &si, uint32_t blk0, uint32_t nv, uint32_t lane,
                                           uint4 (&f)[2 * 4]) {
    const uint4 *pay = reinterpret_cast<const uint4 *>(si.stream + si.po);
    const uint32_t p = lane & 3;
    static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        constexpr int kSel = k | k << 2 | k << 4 | k << 6;   // quad_perm k, k, k, k
        const uint32_t b_o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)blk0, kSel, 0xf, 0xf, false);
        const uint32_t last = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)nv, kSel, 0xf, 0xf, false) - 1;
        f[2 * k] = pay[b_o + min(p, last)];
        f[2 * k + 1] = pay[b_o + min(4 + p, last)];
    });
}

// The blocks of issue_fill into their owners' ring columns: block b = 4 h + p
// of lane 4 j + k goes to rows 4 b + 1 .. 4 b + 4 of that lane's column, with
// row 33 repeating row 1 and row 0 repeating row 32.  A lane writes other
// lanes' columns here; the wave's LDS operations complete in order, so the
// owners' later reads see the writes.
__device__ __forceinline__ void write_fill(uint32_t rbase, uint32_t lane, const uint4 (&f)[2 * 4]) {
    const uint32_t p = lane & 3;
    static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        const uint32_t col = rbase + 4 * k - 4 * p;   // lane 4 j + k's column
        static_for<0, 2>([&](auto hc) __attribute__((always_inline)) {
            constexpr int h = decltype(hc)::value;
            lds_u32 *q = (lds_u32 *)(size_t)(col + (16 * h + 4 * p + 1) * kRowBytes);
            const uint4 v = f[2 * k + h];
            q[0] = v.x;
            q[64] = v.y;
            q[128] = v.z;
            q[192] = v.w;
        });
        if (p == 0) *(lds_u32 *)(size_t)(col + (kRingRows + 1) * kRowBytes) = f[2 * k].x;
        if (p == 3) *(lds_u32 *)(size_t)col = f[2 * k + 1].w;
    });
}

// Two blocks (8 words) into one quarter q of a lane's ring: blocks 8m + 2q
// and 8m + 2q + 1 hold words 32m + 8q .. + 7, rows 8q + 1 .. 8q + 8 (row 32
// is row 0's copy, so the last word of quarter 3 also goes to row 0; the
// first word of quarter 0 also goes to row 33, the copy of row 1).
__device__ __forceinline__ void write_quarter(uint32_t rbase, uint32_t q, const uint4 (&v)[kBatch]) {
    lds_u32 *p = (lds_u32 *)(size_t)(rbase + (8 * q + 1) * kRowBytes);
    static_for<0, kBatch>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        p[(4 * k + 0) * 64] = v[k].x;
        p[(4 * k + 1) * 64] = v[k].y;
        p[(4 * k + 2) * 64] = v[k].z;
        p[(4 * k + 3) * 64] = v[k].w;
    });
    if (q == 0 || q == 3) {
        lds_u32 *e = (lds_u32 *)(size_t)(rbase + (q == 3 ? 0u : 33u) * kRowBytes);
        e[0] = q == 3 ? v[kBatch - 1].w : v[0].x;
    }
}

// Blocks first and first + 1 of a lane's sub-chunk into a refill buffer
// (the second clamped to the lane's last block); a lane with no block left
// there loads the payload's first block instead, the same for every such lane
// (one request).  Returns the buffer's tag: first, or kNone.
__device__ __forceinline__ uint32_t issue_batch(const StreamInfo &si, uint32_t blk0, uint32_t nv, uint32_t first,
                                                uint4 (&v)[kBatch]) {
    const uint4 *pay = reinterpret_cast<const uint4 *>(si.stream + si.po);
    const bool need = first < nv;
    const uint32_t b0 = need ? blk0 + first : 0;
    const uint32_t b1 = need ? blk0 + min(first + 1, nv - 1) : 0;
    v[0] = pay[b0];
    v[1] = pay[b1];
    return need ? first : kNone;
}

// 16 bytes of decoded output, stored with the streaming (non-temporal) hint:
// nothing reads them again in this kernel.
__device__ __forceinline__ void stream_store(uint8_t *p, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = {x, y, z, w};
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(p));
}

// Lane i's 64-byte output piece of a run (a half line) as four 16-byte parts
// o[4 s .. 4 s + 3], turned around within each group of four lanes:
// afterwards part k of lane i holds part i of the piece of lane k of its
// group, so that store k of the group writes one whole 64-byte piece (4 lanes
// x 16 bytes) and a store instruction writes sixteen such pieces instead of
// 16 bytes of 64 lines: partial lines cost L2 extra write-backs (64 MiB
// written 16 bytes a line at a time takes 25 us, 64 bytes at a time 14 us).
// Two butterfly stages exchange parts with lane i ^ d (d = 1, 2) through a
// quad permute: a lane whose bit d is clear keeps its parts s with s & d
// clear and takes the partner's others, and the reverse.
__device__ __forceinline__ void transpose4(uint32_t (&o)[16], uint32_t lane) {
    static_for<0, 2>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = 1 << decltype(dc)::value;
        constexpr int kSel = d == 1 ? 0xb1 : 0x4e;   // quad_perm 1,0,3,2 / 2,3,0,1
        const bool hi = (lane & d) != 0;
        static_for<0, 4>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s0 = decltype(sc)::value;
            if constexpr ((s0 & d) == 0) {
                constexpr int s1 = s0 | d;
                static_for<0, 4>([&](auto wc) __attribute__((always_inline)) {
                    constexpr int w = decltype(wc)::value;
                    const uint32_t x = hi ? o[4 * s0 + w] : o[4 * s1 + w];
                    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kSel, 0xf, 0xf, false);
                    if (hi)
                        o[4 * s0 + w] = y;
                    else
                        o[4 * s1 + w] = y;
                });
            }
        });
    });
}

// Everything the ring did not decode, behind a call, read straight from
// global memory: a segment's last, shorter run; runs that outran the ring
// (long codes); sub-chunks without bits.
template <int CODEC, int PAIRS>
__device__ __noinline__ void decode_rest(const LaneTask &L, const uint32_t *payload, uint64_t pb, uint8_t *dst,
                                         const void *l1, const uint8_t *symtab, const DeepTables *dt,
                                         uint32_t max_len, uint32_t lens, uint32_t k_eg, uint32_t *status) {
    uint32_t bad = 0;
    uint64_t end_pos = 1, want_pos = 0;
    if (L.nv > 0) {   // (symbols but no bits: corrupt)
        GlobalBits S;
        S.init(payload, pb >> 2, L.sb);
        Codes<CODEC, PAIRS, GlobalBits> D(S, l1, symtab, dt, max_len, lens, k_eg);
        if (L.cnt == kSub) {
            for (uint32_t i = 0; i < kSub / 16; ++i) {
                uint32_t o[4];
                D.eight(o[0], o[1]);
                D.eight(o[2], o[3]);
                *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            for (uint32_t k = 0; k < L.cnt; ++k) dst[k] = (uint8_t)D.one();
        }
        bad = D.bad;
        end_pos = S.bit();
        want_pos = L.eb;
    }
    bool pad = false;
    if (end_pos == want_pos && L.pad_end > L.eb) pad = padding_set(payload, L.eb, L.pad_end);
    if ((bad & ~0xffu) || end_pos != want_pos || pad) or_status(status, EC_S_CORRUPT);
}

// Persistent workgroups, one per CU.  A task is one run of 64 consecutive
// sub-chunks for one wave.
//   One stream: the runs are dealt wave by wave over the whole grid: in
//   round r, wave w of workgroup b takes run r * G * 16 + w * G + b (G
//   workgroups), so a partial round still spreads over every CU.
//   Several streams: workgroup-tasks of 16 consecutive runs of one stream
//   (one per wave); workgroup b takes a range of consecutive tasks, which
//   mostly lie in one stream, so the header is checked once, the tables stay
//   in LDS, and each next task's index entries are in flight during a run.
template <int CODEC, int PAIRS>
__global__ __launch_bounds__(64 * waves_for<CODEC>()) void decode_kernel(const DecodeArgs a) {
    constexpr int kWaves = waves_for<CODEC>();
    constexpr int kThreads = 64 * kWaves;
    constexpr uint32_t kTableVec = CODEC == EC_CODEC_QLC       ? kL1Size * 4 / 16
                                   : CODEC == EC_CODEC_HUFFMAN ? kHuffSize * 2 / 16
                                                               : 1;
    constexpr bool kSym = CODEC != EC_CODEC_QLC;
    constexpr bool kHasDeep = CODEC == EC_CODEC_HUFFMAN;
    struct Head {
        uint4 tabv[kTableVec];                 // QLC (u32 entries) / Huffman (u16 entries) decode table
        uint8_t symtab[kSym ? 256 : 4];        // EG: rank -> byte; Huffman: canonical order -> byte
        DeepTables deep[kHasDeep ? 1 : 0];     // Huffman only
    };
    struct Smem {
        Head h;
        alignas(256) uint32_t ring[kWaves][kRegionRows * 64];
    };
    static_assert(sizeof(Smem) <= kLdsBytes, "LDS budget");
    __shared__ Smem sm;
    const void *l1 = sm.h.tabv;
    uint8_t *symtab = sm.h.symtab;
    // (the wave index is uniform: kept in a scalar register, so that run
    // and stream positions derived from it are too)
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t G = gridDim.x, b = blockIdx.x;
    const uint32_t R = (a.blocks_per_seg + 63) / 64;        // runs per stream
    const bool one_stream = a.n_seg == 1;
    const uint32_t Q = (R + kWaves - 1) / kWaves;           // workgroup-tasks per stream (several streams)
    const uint32_t n_u = one_stream ? (R + G * kWaves - 1) / (G * kWaves) * G : Q * a.n_seg;
    // this workgroup's tasks: u_begin, u_begin + u_step, ... below u_end
    const uint32_t per_wg = (n_u + G - 1) / G;
    const uint32_t u_begin = one_stream ? b : b * per_wg, u_step = one_stream ? G : 1u;
    const uint32_t u_end = one_stream ? n_u : min(n_u, u_begin + per_wg);
    // stream and run of this wave in workgroup-task u (run >= R: none)
    auto seg_of = [&](uint32_t u) __attribute__((always_inline)) { return one_stream ? 0u : u / Q; };
    auto run_of = [&](uint32_t u) __attribute__((always_inline)) -> uint32_t {
        if (one_stream) return (u / G) * G * kWaves + wave * G + b;
        return (u - (u / Q) * Q) * kWaves + wave;
    };
    const uint32_t rbase = (uint32_t)(size_t)(lds_u32 *)sm.ring[wave] + 4 * lane;

    uint32_t cur_seg = ~0u;
    StreamInfo si = {};
    const DevTables *tab = nullptr;
    uint32_t *status = nullptr;
    // codebook constants, read once per segment
    uint32_t seg_lens = 0, seg_max_len = 0, seg_k_eg = 0;
    bool seg_ok = false, have_next = false, have_first = false;
    IndexRaw next_raw = {}, first_raw = {};

    for (uint32_t u = u_begin; u < u_end; u += u_step) {
        const uint32_t seg = seg_of(u);
        if (seg != cur_seg) {
            // Streams coded with the codebook already in LDS (a batch with one
            // codebook) keep it: no copy and no barrier.  Uniform over the
            // workgroup.
            const DevTables *seg_tab = seg_tables<DecodeArgs>(seg);
            const bool reload = seg_tab != tab;
            if (reload && tab) __syncthreads();   // the previous segment's tables are no longer read
            tab = seg_tab;
            // the table's 16-bit entries as stored; QLC's are widened to 32
            // bits in LDS (a 16-bit LDS read costs a mask at every use)
            constexpr uint32_t kSrcVec = CODEC == EC_CODEC_QLC ? kL1Size * 2 / 16 : kTableVec;
            constexpr int kTabPer = (kSrcVec + kThreads - 1) / kThreads;
            uint4 tv[kTabPer];
            const uint4 *tsrc = reinterpret_cast<const uint4 *>(CODEC == EC_CODEC_HUFFMAN ? tab->hl1 : tab->l1);
#pragma unroll
            for (int k = 0; k < kTabPer; ++k) {
                if (reload && CODEC != EC_CODEC_EXP_GOLOMB && tid + k * kThreads < kSrcVec) tv[k] = tsrc[tid + k * kThreads];
            }
            const uint8_t *stream = a.in + (uint64_t)seg * a.in_stride;
            status = a.status ? a.status + seg : nullptr;
            seg_lens = tab->qlc_lens;
            seg_max_len = tab->max_len;
            seg_k_eg = (uint32_t)tab->eg_k;
            // every wave reads and checks the header itself (no wait on a barrier)
            const uint64_t *h = reinterpret_cast<const uint64_t *>(stream);
            const uint64_t h0 = h[0], n = h[1], h2 = h[2], po = h[3], pb = h[4], id = h[5];
            const uint32_t magic = (uint32_t)h0, version = (uint32_t)(h0 >> 32) & 0xffffu;
            const uint32_t codec = (uint32_t)(h0 >> 48) & 0xffu, flags = (uint32_t)(h0 >> 56);
            const uint32_t C = (uint32_t)h2, nch = (uint32_t)(h2 >> 32);
            uint32_t bits = 0;
            if (magic != kMagic || version != kVersion || (flags & ~1u)) {
                bits = EC_S_BAD_HEADER;
            } else if (codec != (uint32_t)CODEC || codec != tab->codec || id != tab->codebook_id) {
                bits = EC_S_CODEBOOK_MISMATCH;
            } else if (n != a.seg_n || C == 0 || (C % kSub) || C > kMaxChunk || (uint64_t)nch != (n + C - 1) / C) {
                bits = EC_S_BAD_HEADER;
            } else {
                uint64_t end = kHeaderBytes + 8ull * (nch + 1) + 4ull * nch * (C / kSub) + ((flags & 1) ? 256 : 0);
                end = (end + 255) / 256 * 256;
                if (po != end || pb % 16 || po + pb > a.in_len || (n > 0 && pb == 0) || pb >= (1ull << 36))
                    bits = EC_S_BAD_HEADER;
            }
            // once per segment: by its first workgroup-task's thread 0
            const bool first_u = one_stream ? u == 0 : u == seg * Q;
            if (bits && first_u && tid == 0) flag(status, bits);
            seg_ok = bits == 0;
            cur_seg = seg;
            si.stream = stream;
            si.po = po;
            si.pb = pb;
            si.nch = nch;
            si.spc = C / kSub;
            have_next = false;
            // this wave's first index entries, in flight across the barrier
            const uint32_t run0 = run_of(u);
            have_first = seg_ok && run0 < R;
            if (have_first) first_raw = issue_index(a, si, run0 * 64 + lane);
            if (reload) {
#pragma unroll
                for (int k = 0; k < kTabPer; ++k) {
                    const uint32_t i = tid + k * kThreads;
                    if (CODEC == EC_CODEC_QLC && i < kSrcVec) {
                        const uint4 v = tv[k];
                        sm.h.tabv[2 * i] = make_uint4(v.x & 0xffffu, v.x >> 16, v.y & 0xffffu, v.y >> 16);
                        sm.h.tabv[2 * i + 1] = make_uint4(v.z & 0xffffu, v.z >> 16, v.w & 0xffffu, v.w >> 16);
                    } else if (CODEC == EC_CODEC_HUFFMAN && i < kSrcVec) {
                        sm.h.tabv[i] = tv[k];
                    }
                }
                if constexpr (kSym) {
                    if (tid < 256) symtab[tid] = tab->sym[tid];
                }
                if constexpr (CODEC == EC_CODEC_HUFFMAN) {
                    constexpr uint32_t kDeep = EC_MAX_CODE_LEN - kHuffBits;
                    if (tid < kDeep) {
                        sm.h.deep[0].limit[tid] = tab->limit[kHuffBits + 1 + tid];
                        sm.h.deep[0].first_code[tid] = tab->first_code[kHuffBits + 1 + tid];
                        sm.h.deep[0].first_idx[tid] = tab->first_idx[kHuffBits + 1 + tid];
                    }
                }
                __syncthreads();
            }
        }
        if (!seg_ok) continue;   // uniform over the workgroup

        const uint32_t run = run_of(u);
        const uint32_t g0 = run * 64;   // the wave's first sub-chunk
        if (run >= R) {                 // uniform over the wave
            have_next = false;
            continue;
        }
        // Issue priority follows progress: a wave sets the highest level for
        // its task's setup and fill, then one level lower for each group of
        // 64 symbols it finishes.  Without it the SIMD's arbiter favours the
        // oldest wave, which starves the younger waves' setup while it
        // decodes (their fills wait up to 15 us) and leaves one wave per
        // SIMD decoding alone at the end.
        __builtin_amdgcn_s_setprio(3);
        const LaneTask L = resolve(a, si, have_next ? next_raw : have_first ? first_raw : issue_index(a, si, g0 + lane),
                                   g0 + lane, status);
        have_first = false;
        const bool live = L.ok && L.cnt > 0;   // L.nv == 0 then means a sub-chunk without bits: corrupt
        const bool full = live && L.cnt == kSub && L.nv > 0;
        // the next task's index entries, in flight during this run
        const uint32_t u1 = u + u_step;
        const uint32_t run1 = u1 < u_end ? run_of(u1) : R;
        have_next = u1 < u_end && seg_of(u1) == seg && run1 < R;
        uint8_t *const wave_out = a.out + (uint64_t)seg * a.out_stride + (uint64_t)g0 * kSub;
        const uint32_t *payload = reinterpret_cast<const uint32_t *>(si.stream + si.po);
        if (__ballot(full) != ~0ull) {
            // a segment's last, shorter run, or an index found corrupt: every
            // live lane decodes from global memory
            if (have_next) next_raw = issue_index(a, si, run1 * 64 + lane);
            if (live)
                decode_rest<CODEC, PAIRS>(L, payload, si.pb, wave_out + lane * kSub, l1, symtab, sm.h.deep,
                                          seg_max_len, seg_lens, seg_k_eg, status);
            asm volatile("" ::: "memory");
            continue;
        }
        // what the end of the run needs, relative to the lane's first block
        const uint32_t blk0 = (uint32_t)L.blk0;   // payloads are below 2^36 bytes
        const uint32_t nv = L.nv;
        const uint32_t start = (uint32_t)(L.sb - L.blk0 * 128);
        const uint32_t want = (uint32_t)(L.eb - L.blk0 * 128);
        const uint32_t pad_to = L.pad_end > L.eb ? (uint32_t)(L.pad_end - L.blk0 * 128) : 0u;
        // the ring's eight blocks, then the next task's index (loaded in
        // every case, from this run's entries when there is no next task, so
        // that the fill's wait never covers it), then the fill into the ring;
        // the refill buffers start empty
        uint4 f[2 * 4];
        issue_fill(si, blk0, nv, lane, f);
        next_raw = issue_index(a, si, (have_next ? run1 : run) * 64 + lane);
        write_fill(rbase, lane, f);
        uint4 bufA[kBatch], bufB[kBatch];
        uint32_t tagA = kNone, tagB = kNone;
        uint32_t nb = 8;   // blocks written so far
        // the wave's LDS operations complete in program order
        asm volatile("" ::: "memory");

        RingBits S;
        S.rbase = rbase;
        S.Y = 31 + start;
        bool over = false;   // the run consumed bits the ring did not hold yet
        uint32_t bad = 0;
        // store k of a group's output: lane 4 j + p writes part p of the piece
        // of lane 4 j + k (see transpose4)
        const uint32_t part = (lane & ~3u) * kSub + 16 * (lane & 3);
        constexpr int kOW = 16;   // words per group: a 64-byte piece per lane
        static_assert(kSub / (4 * kOW) <= 4, "one issue priority level per group");
        uint32_t o[kOW];
        auto store_part = [&](int grp, auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            stream_store(wave_out + part + (4 * kOW * grp + k * kSub), o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
        };
        {
            Codes<CODEC, PAIRS, RingBits> D(S, l1, symtab, sm.h.deep, seg_max_len, seg_lens, seg_k_eg);
            // A group is 64 symbols: four passes of 16, pass p into o[4 p ..],
            // each followed by a refill point.  Output leaves one 16-byte store
            // per point: the previous group's parts 1, 2, 3 at points 0, 1, 2
            // (before passes 1, 2, 3 reuse their registers), and at point 3,
            // after the group's turn-around, its own part 0.  Every point so
            // issues one store and then its two loads, and a buffer's loads
            // are followed by exactly three memory operations (two before the
            // first group's stores begin) when its turn comes two points
            // later: the wait at each point is exact and never covers the
            // loads or stores of the point just before.
            static_for<0, kSub / (4 * kOW)>([&](auto gc) __attribute__((always_inline)) {
                constexpr int grp = decltype(gc)::value;
                __builtin_amdgcn_s_setprio(3 - grp);
                // vmcnt <= 2 (expcnt and lgkmcnt left at their maxima): the
                // other buffer's two loads may still be in flight (a store
                // may complete after later loads, so stores are not counted)
                constexpr int kWait = 0x0f72;
                // 16 symbols -> o[8 i + 4 P ..], chosen by value: every index
                // into o is a constant (an index chosen at run time would move
                // o to memory)
                auto pass = [&](int i, auto pc) __attribute__((always_inline)) {
                    constexpr int P = decltype(pc)::value;
                    uint32_t w[4];
                    D.eight(w[0], w[1]);
                    D.eight(w[2], w[3]);
                    static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
                        constexpr int k = decltype(kc)::value;
                        o[4 * P + k] = i == 0 ? w[k] : o[4 * P + k];
                        o[8 + 4 * P + k] = i == 0 ? o[8 + 4 * P + k] : w[k];
                    });
                };
                // A refill point with buffer X (the other one: Y): check the
                // position against the blocks written; write X if it holds
                // blocks (always the next ones, with room: see the load
                // condition); store; reload X with the next blocks Y does not
                // hold when the ring has room for them now, and so two
                // points later.
                auto refill = [&](uint4(&X)[kBatch], uint32_t &tagX, uint32_t tagY, auto &&store)
                                  __attribute__((always_inline)) {
                    const uint32_t pos = S.bit();
                    over = over || pos > nb * 128;
                    if (tagX == nb) {
                        __builtin_amdgcn_s_waitcnt(kWait);
                        write_quarter(rbase, (nb >> 1) & 3, X);
                        nb += kBatch;
                    }
                    store();
                    const uint32_t next = tagY == nb ? nb + kBatch : nb;
                    const bool room = next + kBatch <= (pos >> 7) + kRingBlocks;
                    tagX = issue_batch(si, blk0, nv, room ? next : kNone, X);
                };
                // the parts a point may store, read at fixed indexes and
                // chosen by value (a choice of index would move o to memory)
                auto part_of = [&](auto kc) __attribute__((always_inline)) {
                    constexpr int k = decltype(kc)::value;
                    return make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
                };
                // one of two parts, chosen word by word
                auto put = [&](uint32_t off, bool first, const uint4 &v, const uint4 &w) __attribute__((always_inline)) {
                    stream_store(wave_out + part + off, first ? v.x : w.x, first ? v.y : w.y, first ? v.z : w.z,
                                 first ? v.w : w.w);
                };
                // two passes of 16 symbols per iteration, a refill point
                // after each: the buffers' turns are fixed in the code
#pragma nounroll
                for (int i = 0; i < kOW / 8; ++i) {
                    pass(i, std::integral_constant<int, 0>{});
                    refill(bufA, tagA, tagB, [&]() __attribute__((always_inline)) {
                        if constexpr (grp > 0) {
                            // the previous group's part 1 (first step) or 3
                            const uint4 p1 = part_of(std::integral_constant<int, 1>{});
                            const uint4 p3 = part_of(std::integral_constant<int, 3>{});
                            put(4 * kOW * (grp - 1) + (i == 0 ? 1 : 3) * kSub, i == 0, p1, p3);
                        }
                    });
                    pass(i, std::integral_constant<int, 1>{});
                    refill(bufB, tagB, tagA, [&]() __attribute__((always_inline)) {
                        // first step: the previous group's part 2; second:
                        // this group, turned around, its part 0
                        if (i != 0) transpose4(o, lane);
                        const uint4 p2 = part_of(std::integral_constant<int, 2>{});
                        const uint4 p0 = part_of(std::integral_constant<int, 0>{});
                        if (grp > 0 || i != 0) put(i == 0 ? 4 * kOW * (grp - 1) + 2 * kSub : 4 * kOW * grp, i == 0, p2, p0);
                    });
                }
            });
            constexpr int kLast = kSub / (4 * kOW) - 1;
            store_part(kLast, std::integral_constant<int, 1>{});
            store_part(kLast, std::integral_constant<int, 2>{});
            store_part(kLast, std::integral_constant<int, 3>{});
            bad = D.bad;
        }
        __builtin_amdgcn_s_setprio(0);
        const uint32_t end = S.bit();
        over = over || end > nb * 128;
        bool corrupt = !over && ((bad & ~0xffu) || end != want);
        // the zero padding after a chunk's last sub-chunk
        const bool pad_check = !over && !corrupt && pad_to != 0;
        if (__ballot(pad_check))
            if (pad_check) corrupt = padding_set(payload, (uint64_t)blk0 * 128 + want, (uint64_t)blk0 * 128 + pad_to);
        if (__ballot(over)) {
            // a lane that outran its ring rewrites the line its group stored
            // for it: the group's stores complete first
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            if (over) {
                LaneTask T;
                T.sb = (uint64_t)blk0 * 128 + start;
                T.eb = (uint64_t)blk0 * 128 + want;
                T.pad_end = pad_to ? (uint64_t)blk0 * 128 + pad_to : 0;
                T.first_sym = (uint64_t)(g0 + lane) * kSub;
                T.blk0 = blk0;
                T.nv = nv;
                T.cnt = kSub;
                T.ok = true;
                decode_rest<CODEC, PAIRS>(T, payload, si.pb, wave_out + lane * kSub, l1, symtab, sm.h.deep,
                                          seg_max_len, seg_lens, seg_k_eg, status);
            }
        }
        // one status update per wave (a same-address atomic per lane of a
        // corrupt stream would serialise 64 times over)
        const uint64_t bad_lanes = __ballot(corrupt);
        if (bad_lanes && lane == (uint32_t)__builtin_ctzll(bad_lanes)) flag(status, EC_S_CORRUPT);
        // the ring is rewritten at the next task, after this lane's reads
        asm volatile("" ::: "memory");
    }
}

template <int CODEC, int PAIRS>
hipError_t launch_one(const DecodeArgs &a, hipStream_t s) {
    constexpr int kWaves = waves_for<CODEC>();
    constexpr int kThreads = 64 * kWaves;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<CODEC, PAIRS>, kThreads, 0);
    if (e != hipSuccess) return e;
    const uint32_t R = (a.blocks_per_seg + 63) / 64;
    // one stream: up to one workgroup per run (its waves dealt over the grid);
    // several: up to one per workgroup-task
    uint64_t cap = a.n_seg == 1 ? R : (uint64_t)(R + kWaves - 1) / kWaves * a.n_seg;
    if (cap == 0) cap = 1;   // still validate the header
    const uint64_t resident = (uint64_t)(per_cu > 0 ? per_cu : 1) * (uint64_t)(cus > 0 ? cus : 1);
    const uint32_t grid = (uint32_t)(cap < resident ? cap : resident);
    hipLaunchKernelGGL((decode_kernel<CODEC, PAIRS>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, uint32_t codec, uint32_t max_len, hipStream_t s) {
    switch (codec) {
        case EC_CODEC_QLC:
            return launch_one<EC_CODEC_QLC, 1>(a, s);        // codes <= 11 bits
        case EC_CODEC_HUFFMAN:
            return launch_one<EC_CODEC_HUFFMAN, 1>(a, s);    // pairs when they fit, else one per window
        default:
            if (max_len <= 16) return launch_one<EC_CODEC_EXP_GOLOMB, 1>(a, s);
            return launch_one<EC_CODEC_EXP_GOLOMB, 0>(a, s);
    }
}

}  // namespace ec
