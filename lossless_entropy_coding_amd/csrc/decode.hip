// Chunk-parallel decoder.
//
// Every 256-symbol sub-chunk starts at a bit offset recorded in the stream
// index, so one lane decodes one sub-chunk serially and a wave64 decodes 64
// sub-chunks side by side.  Each lane first copies the 16-byte blocks that
// hold its sub-chunk from the payload into its own column of the wave's LDS
// region: word k of lane l's bits goes to row k, column l.  A 64-bit window
// at any bit position is then one read of three rows of the lane's column
// plus two funnel shifts, and the 64 lanes of a read always hit 64 different
// banks, whatever their positions (a contiguous copy of the compressed span
// has the lanes read at scattered addresses: about twice the LDS time in bank
// conflicts).  One window serves four codes.  (A global load inside the
// decode loop would stall on the output stores too: one counter tracks both.)
// QLC and EG stage the whole sub-chunk at once.  Huffman stages it in two
// halves of a shorter column (the blocks still unread move down at the
// half-run point), so that twelve waves per CU fit the LDS instead of eight:
// its loop mostly waits on LDS reads, and more waves in flight hide them.
// A sub-chunk too long for the region (data that barely compresses) is
// decoded straight from global memory.
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
// After its last symbol a lane checks that it stopped exactly where the index
// says its sub-chunk ends.
#include "dev_common.h"

namespace ec {

namespace {

// Waves of the one workgroup per CU (which shares one copy of the tables):
// three per SIMD for Huffman codes (its decode loop fits 168 VGPRs and
// waits mostly on LDS), else two.
template <int CODEC>
constexpr int waves_for() {
    return CODEC == EC_CODEC_HUFFMAN ? 12 : 8;
}
constexpr uint32_t kLdsBytes = 160 * 1024;
constexpr uint32_t kRowBytes = 64 * 4;               // one word per lane
// Rows past the last region that a lane may read: a position is clamped to
// its region at the start of every 8 codes, which then move it by at most
// 8 codes of the longest length the codec can read (QLC 11 bits, EG 25,
// Huffman 40), and a window reads up to three rows from there.
template <int CODEC>
constexpr uint32_t guard_rows() {
    constexpr uint32_t kMaxCode = CODEC == EC_CODEC_QLC ? 11 : CODEC == EC_CODEC_HUFFMAN ? EC_MAX_CODE_LEN : 25;
    return (8 * kMaxCode + 31) / 32 + 3;
}

// Bits of a lane's sub-chunk staged in its LDS column.  Row r of the wave's
// region holds word r - 1 of every lane's bits (row 0 is never written: a
// window at a word boundary reads it and shifts it out).  Y is the position
// plus 31 plus the region's row offset in bits (its LDS byte address / 8), so
// the row holding the bit before the position is Y >> 5 and its LDS byte
// address is (Y >> 5) * 256 + 4 * lane: no base to add, and a 32-bit window
// never needs a special case.  A valid sub-chunk never leaves its region;
// for corrupt streams prepare() clamps the position to the region's last row
// every 8 codes, so reads stay inside the allocation (rows past a lane's data
// hold other data or guard rows) and the end check flags the stream.
struct ColBits {
    uint32_t Y;      // see above
    uint32_t col;    // 4 * lane
    uint32_t base;   // Y of the lane's bit 0
    uint32_t ylim;   // largest Y in the region's last row

    typedef __attribute__((address_space(3))) const uint32_t lds_word;
    __device__ __forceinline__ uint32_t at(uint32_t yy) const {
        lds_word *w = (lds_word *)(size_t)(((yy >> 5) << 8) | col);
        return __builtin_amdgcn_alignbit(w[0], w[64], ~yy);
    }
    __device__ __forceinline__ uint32_t win() const { return at(Y); }
    __device__ __forceinline__ uint64_t win64() const {   // rows k, k + 1, k + 2 of the column
        lds_word *w = (lds_word *)(size_t)(((Y >> 5) << 8) | col);
        const uint32_t d0 = w[0], d1 = w[64], d2 = w[128];
        return ((uint64_t)__builtin_amdgcn_alignbit(d0, d1, ~Y) << 32) | __builtin_amdgcn_alignbit(d1, d2, ~Y);
    }
    __device__ __forceinline__ void adv(uint32_t l) { Y += l; }
    __device__ __forceinline__ void prepare() { Y = min(Y, ylim); }
    __device__ __forceinline__ uint64_t bit() const { return Y - base; }   // lane-relative position
};

// Bits of a lane's sub-chunk read straight from global memory (spans that
// do not fit in LDS): a 64-bit MSB-aligned buffer refilled 32 bits at a time,
// loads clamped to the payload.
struct GlobalBits {
    const uint32_t *base;   // lane's first payload word
    uint32_t last;          // last readable word, relative to base
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
        last = (uint32_t)(lastw - b);
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
// of the decode table's entries.
__device__ __noinline__ uint32_t huff_deep(uint64_t window, const DeepTables *dt, const uint8_t *sym, uint32_t mx) {
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

// Decode one 256-symbol run (or the cnt < 256 symbols of a segment's last
// run) from source S into dst; returns the bits of the QLC / EG "not a
// codeword" flags (bit 8 and up).  FULL > 0: half HALF (symbols
// 128 * HALF ..; 2: both halves) of a whole run from an LDS column (the
// common case), in code with a fixed number of stores, so that the compiler
// can count the memory operations in flight across it.
template <int CODEC, int PAIRS, int FULL, class Src, int HALF = 0>
__device__ __forceinline__ uint32_t decode_run(Src &S, uint32_t cnt, uint8_t *dst, const uint16_t *l1,
                                               const uint8_t *symtab, const DeepTables *dt, uint32_t max_len,
                                               uint32_t lens, uint32_t k_eg) {
    uint32_t bad = 0;
    // QLC code lengths by area, one byte each: areas 0-3 in llo, 4-7 in lhi
    uint32_t llo = 0, lhi = 0;
    if (CODEC == EC_CODEC_QLC) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            llo |= ((lens >> (4 * k)) & 15u) << (8 * k);
            lhi |= ((lens >> (4 * k + 16)) & 15u) << (8 * k);
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
    auto code_at = [&](uint32_t w) __attribute__((always_inline)) -> Code {
        if (CODEC == EC_CODEC_QLC) {
            const uint32_t sel = __builtin_amdgcn_alignbit(0x01818180u, w, 29);   // 0x0c0c0c00 | w >> 29
            return Code{l1[w >> 21], __builtin_amdgcn_perm(lhi, llo, sel)};
        } else if (CODEC == EC_CODEC_HUFFMAN) {
            uint32_t e = l1[w >> (32 - kHuffBits)];
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
    };
    // the symbol of an entry, and the byte permute that takes the symbols of
    // two entries (first in byte 0, second in byte 1)
    constexpr uint32_t kSymShift = CODEC == EC_CODEC_HUFFMAN ? 8 : 0;
    constexpr uint32_t kPairSel = CODEC == EC_CODEC_HUFFMAN ? 0x0c0c0501u : 0x0c0c0400u;
    auto one = [&]() __attribute__((always_inline)) -> uint32_t {
        const Code c = code_at(S.win());
        if (CODEC == EC_CODEC_QLC) bad |= c.e;
        S.adv(c.len);
        return (c.e >> kSymShift) & 0xffu;
    };
    // two codes from one window when both fit in it; returns byte0 | byte1 << 8
    auto two = [&]() __attribute__((always_inline)) -> uint32_t {
        const uint32_t w = S.win();
        Code c1, c2;
        if (CODEC != EC_CODEC_HUFFMAN) c1 = code_at(w);
        if (CODEC == EC_CODEC_HUFFMAN) {
            // Both table reads from the one window: a code the table covers
            // has at most 13 bits, so 19 bits of the window follow it.  A
            // longer code (rare) sends the lanes that hold one to the
            // canonical search and a fresh window for the second code.
            // (shifts take their amount modulo 32: a shift by the entry is
            // a shift by the code's length)
            uint32_t e1 = l1[w >> (32 - kHuffBits)];
            uint32_t e2 = l1[(w << (e1 & 31u)) >> (32 - kHuffBits)];
            if (min(e1, e2) == 0u) {
                if (e1 == 0u) e1 = huff_deep(S.win64(), dt, symtab, max_len);
                S.adv(e1 & 0xffu);
                e2 = l1[S.win() >> (32 - kHuffBits)];
                if (e2 == 0u) e2 = huff_deep(S.win64(), dt, symtab, max_len);
                S.adv(e2 & 0xffu);
            } else {
                S.adv((e1 + e2) & 0xffu);   // lengths of at most 13 bits: no carry into the symbols
            }
            c1.e = e1;
            c2.e = e2;
        } else {
            c2 = code_at(w << c1.len);
            S.adv(c1.len + c2.len);
            if (CODEC == EC_CODEC_QLC) bad |= c1.e | c2.e;
        }
        return __builtin_amdgcn_perm(c2.e, c1.e, kPairSel);   // c1's symbol, c2's symbol
    };
    // Four codes from one 64-bit window: the second pair's 32-bit window lies
    // inside the 64 bits when a pair has at most 32 bits (QLC: codes of at
    // most 11 bits; EG in pair mode: at most 16; Huffman: codes the table
    // covers, at most 13 bits each, else (rare) the pair step twice).
    // Returns the four bytes in order.
    auto four = [&]() __attribute__((always_inline)) -> uint32_t {
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
        const uint32_t e1 = l1[w >> (32 - kHuffBits)];
        const uint32_t e2 = l1[(w << (e1 & 31u)) >> (32 - kHuffBits)];
        const uint32_t e12 = e1 + e2;   // lengths add in the low byte (at most 26)
        const uint32_t v = (uint32_t)((W << (e12 & 63u)) >> 32);
        const uint32_t e3 = l1[v >> (32 - kHuffBits)];
        const uint32_t e4 = l1[(v << (e3 & 31u)) >> (32 - kHuffBits)];
        if (min(min(e1, e2), min(e3, e4)) == 0u) {
            const uint32_t p0 = two(), p1 = two();
            return p0 | (p1 << 16);
        }
        S.adv((e12 + e3 + e4) & 0xffu);
        return __builtin_amdgcn_perm(e2, e1, kPairSel) | (__builtin_amdgcn_perm(e4, e3, kPairSel) << 16);
    };
    // eight codes -> two output words
    auto eight = [&](uint32_t &lo, uint32_t &hi) __attribute__((always_inline)) {
        S.prepare();
        if (FULL && PAIRS) {
            lo = four();
            hi = four();
        } else if (PAIRS) {
            const uint32_t p0 = two(), p1 = two(), p2 = two(), p3 = two();
            lo = p0 | (p1 << 16);
            hi = p2 | (p3 << 16);
        } else {
            uint32_t b[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) b[k] = one();
            lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
            hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        }
    };

    if constexpr (FULL == 2) {
        // A loop of 16 codes a pass (Huffman, EG): the whole run unrolled
        // would not fit the instruction cache next to the Huffman pair step's
        // rare long code path, and the EG loop would spill.  The words of a
        // half run still gather in registers (placed by the uniform pass
        // counter) and leave as one whole 128-byte line per lane: 16-byte
        // stores to 64 lanes' separate lines leave partial lines in L2 that
        // get written back several times.
        static_for<(HALF == 2 ? 0 : HALF), (HALF == 2 ? 2 : HALF + 1)>([&](auto hf) __attribute__((always_inline)) {
            constexpr int half = decltype(hf)::value;
            uint32_t o[32];
#pragma nounroll
            for (int i = 0; i < 8; ++i) {
                uint32_t w0, w1, w2, w3;
                eight(w0, w1);
                eight(w2, w3);
                // a uniform branch per pass keeps o in registers
                static_for<0, 8>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    if (i == j) {
                        o[4 * j] = w0;
                        o[4 * j + 1] = w1;
                        o[4 * j + 2] = w2;
                        o[4 * j + 3] = w3;
                    }
                });
            }
            uint4 *line = reinterpret_cast<uint4 *>(dst + 128 * half);
            static_for<0, 8>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                line[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
            });
        });
    } else if constexpr (FULL == 1) {
        // 128 decoded bytes are collected in registers and written as one
        // whole cache line: 16-byte stores to 64 lanes' separate lines leave
        // partial lines in L2 that get written back more than once
        static_for<(HALF == 2 ? 0 : HALF), (HALF == 2 ? 2 : HALF + 1)>([&](auto hf) __attribute__((always_inline)) {
            constexpr int half = decltype(hf)::value;
            uint32_t o[32];
            static_for<0, 16>([&](auto hc) __attribute__((always_inline)) {
                constexpr int h = decltype(hc)::value;
                eight(o[2 * h], o[2 * h + 1]);
                // keep each group's table reads next to their use (without
                // this the scheduler hoists all 128 symbols' reads and spills)
                __builtin_amdgcn_sched_barrier(0);
            });
            uint4 *line = reinterpret_cast<uint4 *>(dst + 128 * half);
            static_for<0, 8>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                line[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
            });
        });
    } else if (cnt == kSub) {
        for (int i = 0; i < kSub / 16; ++i) {
            uint32_t o[4];
            eight(o[0], o[1]);
            eight(o[2], o[3]);
            *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else {
        for (uint32_t k = 0; k < cnt; ++k) {
            S.prepare();
            dst[k] = (uint8_t)one();
        }
    }
    return bad;
}

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
// loads are in flight while the wave decodes an earlier task).
struct IndexRaw {
    uint64_t co0, co1;        // the lane's chunk: byte offsets of its start and end in the payload
    uint32_t e_start, e_end;  // the lane's sub-chunk: start and end bit in its chunk
    bool last;                // the sub-chunk is its chunk's last: the padding after it is checked
};

// Stream fields the tasks of a segment share (validated once per segment).
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
    r.co0 = chunk_off[c];
    r.co1 = chunk_off[c + 1];
    r.e_end = sub_end[(uint64_t)c * si.spc + j];
    r.e_start = j ? sub_end[(uint64_t)c * si.spc + j - 1] : 0u;
    r.last = j == si.spc - 1 || gl == a.blocks_per_seg - 1;
    return r;
}

// Checks the index entries of sub-chunk g (flags a corrupt index).
__device__ __forceinline__ LaneTask resolve(const DecodeArgs &a, const StreamInfo &si, const IndexRaw &r, uint32_t g,
                                            uint32_t *status) {
    const bool active = g < a.blocks_per_seg;
    LaneTask t;
    t.ok = active && r.co0 <= r.co1 && r.co1 <= si.pb && !(r.co0 & 15) && (uint64_t)r.e_end <= (r.co1 - r.co0) * 8 &&
           r.e_start <= r.e_end;
    if (active && !t.ok) flag(status, EC_S_CORRUPT);
    t.sb = r.co0 * 8 + r.e_start;
    t.eb = r.co0 * 8 + r.e_end;
    t.pad_end = r.last ? r.co1 * 8 : 0;
    t.first_sym = (uint64_t)g * kSub;
    t.cnt = !active ? 0u : (a.seg_n - t.first_sym < kSub ? (uint32_t)(a.seg_n - t.first_sym) : (uint32_t)kSub);
    const bool live = t.ok && t.cnt > 0 && t.eb > t.sb;
    t.blk0 = live ? t.sb >> 7 : 0;
    t.nv = live ? (uint32_t)(((t.eb - 1) >> 7) - t.blk0 + 1) : 0u;
    return t;
}

// Blocks FIRST .. FIRST + K - 1 of a lane's sub-chunk, loaded into
// registers (indexes clamped to the lane's last block, or to the payload's
// first block for lanes with nothing to decode, so every load stays inside
// the payload).
template <int K, int FIRST = 0>
__device__ __forceinline__ void issue_blocks(const StreamInfo &si, const LaneTask &t, uint4 (&v)[K]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(si.stream + si.po) + t.blk0;
    const uint32_t last = t.nv ? t.nv - 1 : 0u;
    static_for<0, K>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        v[k] = src[min((uint32_t)(FIRST + k), last)];
    });
}

// Blocks first .. nv_max - 1 of the lanes' sub-chunks (those not
// prefetched) into their LDS columns, behind a call (whole-run staging).
__device__ __noinline__ void stage_rest(uint32_t col_word0, const uint4 *src, uint32_t nv, uint32_t first,
                                        uint32_t nv_max) {
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    for (uint32_t j = first; j < nv_max; j += 4) {   // four loads in flight per lane
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (j + k < nv) v[k] = src[j + k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (j + k < nv) {
                lds_u32 *w = (lds_u32 *)(size_t)(col_word0 + (4 * (j + k)) * kRowBytes);
                w[0] = v[k].x;
                w[64] = v[k].y;
                w[128] = v[k].z;
                w[192] = v[k].w;
            }
        }
    }
}

// Everything but a whole run decoded from the lane's column, behind a call,
// read straight from global memory: a segment's last, shorter run; runs
// whose halves do not fit the column's stages (data that barely compresses);
// sub-chunks without bits.
template <int CODEC, int PAIRS>
__device__ __noinline__ void decode_rest(const LaneTask &L, const uint32_t *payload, uint64_t pb, uint8_t *dst,
                                         const uint16_t *l1, const uint8_t *symtab, const DeepTables *dt,
                                         uint32_t max_len, uint32_t lens, uint32_t k_eg, uint32_t *status) {
    uint32_t bad = 0;
    uint64_t end_pos = 1, want_pos = 0;
    if (L.nv > 0) {   // (symbols but no bits: corrupt)
        GlobalBits S;
        S.init(payload, pb >> 2, L.sb);
        bad = decode_run<CODEC, PAIRS, 0>(S, L.cnt, dst, l1, symtab, dt, max_len, lens, k_eg);
        end_pos = S.bit();
        want_pos = L.eb;
    }
    bool pad = false;
    if (end_pos == want_pos && L.pad_end > L.eb) pad = padding_set(payload, L.eb, L.pad_end);
    if ((bad & ~0xffu) || end_pos != want_pos || pad) or_status(status, EC_S_CORRUPT);
}

// Persistent workgroups: workgroup b takes tasks b, b + G, ... (G = grid);
// a task is 64 consecutive sub-chunks of one stream per wave.
//
// A lane's column holds kStage blocks at a time, in two stages.  Stage 1
// is the sub-chunk's first kStage blocks (prefetched in registers while the
// wave decoded its previous task); the blocks after them are loaded into
// registers meanwhile.  At the half-run point (128 symbols) the blocks not
// yet consumed move down to the column's first slots and the loaded ones
// follow them (stage 2).  A lane whose first half reads past stage 1, or
// whose rest does not fit stage 2, decodes its run again from global memory.
template <int CODEC, int PAIRS>
__global__ __launch_bounds__(64 * waves_for<CODEC>()) void decode_kernel(const DecodeArgs a) {
    constexpr uint32_t kWaves = waves_for<CODEC>();
    constexpr uint32_t kThreads = 64 * kWaves;
    constexpr uint32_t kTableVec = CODEC == EC_CODEC_QLC       ? kL1Size * 2 / 16
                                   : CODEC == EC_CODEC_HUFFMAN ? kHuffSize * 2 / 16
                                                               : 1;
    constexpr bool kSym = CODEC != EC_CODEC_QLC;
    constexpr bool kHasDeep = CODEC == EC_CODEC_HUFFMAN;
    constexpr uint32_t kGuardRows = guard_rows<CODEC>();
    struct Head {
        uint4 tabv[kTableVec];     // QLC / Huffman decode table
        uint8_t symtab[kSym ? 256 : 4];       // EG: rank -> byte; Huffman: canonical order -> byte
        DeepTables deep[kHasDeep ? 1 : 0];    // Huffman only
    };
    // the rest of the CU's LDS: one region of kRows rows per wave, then guard rows
    constexpr uint32_t kHeadBytes = (sizeof(Head) + kRowBytes - 1) / kRowBytes * kRowBytes;
    constexpr uint32_t kRows = (kLdsBytes - kHeadBytes - kGuardRows * kRowBytes) / (kWaves * kRowBytes);
    // Huffman: two stages of kStage blocks; other codecs: the whole run
    // staged at once (up to kRows rows), kStage blocks of it prefetched
    constexpr bool kTwo = CODEC == EC_CODEC_HUFFMAN;
    constexpr int kStage = kTwo ? (int)((kRows - 1) / 4 < 16 ? (kRows - 1) / 4 : 16) : 16;
    static_assert(kStage >= 8 && (kTwo || 1 + 4 * kStage <= kRows), "column stages too short");
    struct Smem {
        Head h;
        alignas(256) uint32_t cols[kWaves][kRows * 64];
        uint32_t guard[kGuardRows * 64];
    };
    static_assert(sizeof(Smem) <= kLdsBytes, "LDS budget");
    __shared__ Smem sm;
    const uint16_t *l1 = reinterpret_cast<const uint16_t *>(sm.h.tabv);
    uint8_t *symtab = sm.h.symtab;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t gx = (a.blocks_per_seg + kThreads - 1) / kThreads > 0 ? (a.blocks_per_seg + kThreads - 1) / kThreads
                                                                           : 1u;
    const uint32_t n_tasks = gx * a.n_seg;
    // One stream: the last, partial round of tasks (every task, when the
    // grid is larger than the task count) is spread over every workgroup
    // wave by wave (wave w of workgroup b takes the round's (w * G + b)-th
    // run of 64 sub-chunks), so that its waves sit on the SIMDs of all CUs
    // instead of filling a few CUs.
    const uint32_t tail_at = n_tasks / gridDim.x * gridDim.x;   // first task of a partial round
    const bool spread = a.n_seg == 1 && tail_at != n_tasks;
    const uint32_t n_iter = spread ? tail_at + gridDim.x : n_tasks;
    auto seg_of = [&](uint32_t tt) __attribute__((always_inline)) { return spread ? 0u : tt / gx; };
    // the wave's first sub-chunk in task tt
    auto first_sub = [&](uint32_t tt) __attribute__((always_inline)) -> uint32_t {
        if (spread && tt >= tail_at) return tail_at * kThreads + (wave * gridDim.x + blockIdx.x) * 64;
        return (tt - tt / gx * gx) * kThreads + wave * 64;
    };
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    const uint32_t region = (uint32_t)(size_t)(lds_u32 *)sm.cols[wave];   // 256-byte aligned
    lds_u32 *my_col = (lds_u32 *)(size_t)(region + 4 * lane);

    uint32_t cur_seg = ~0u;
    StreamInfo si = {};
    const DevTables *tab = nullptr;
    uint32_t *status = nullptr;
    // codebook constants, read once per segment: a global load in the loop
    // would wait for the prefetch loads issued before it
    uint32_t seg_lens = 0, seg_max_len = 0, seg_k_eg = 0;
    bool have_cur = false, have_next_raw = false, have_first = false, seg_ok = false;
    LaneTask cur = {};
    IndexRaw next_raw = {}, first_raw = {};
    // blocks in flight: during a first half this task's blocks kStage ..,
    // during a second half the next task's first kStage blocks
    uint4 pre[kStage];
#pragma unroll
    for (int k = 0; k < kStage; ++k) pre[k] = make_uint4(0u, 0u, 0u, 0u);

    for (uint32_t t = blockIdx.x; t < n_iter; t += gridDim.x) {
        const uint32_t seg = seg_of(t);
        if (seg != cur_seg) {
            __syncthreads();   // the previous segment's tables are no longer read
            tab = seg_tables<DecodeArgs>(seg);
            // this thread's share of the decode table, in flight while the
            // header is checked and the first task's index entries are requested
            constexpr int kTabPer = (kTableVec + kThreads - 1) / kThreads;
            uint4 tv[kTabPer];
            const uint4 *tsrc = reinterpret_cast<const uint4 *>(CODEC == EC_CODEC_HUFFMAN ? tab->hl1 : tab->l1);
#pragma unroll
            for (int k = 0; k < kTabPer; ++k) {
                if (CODEC != EC_CODEC_EXP_GOLOMB && tid + k * kThreads < kTableVec) tv[k] = tsrc[tid + k * kThreads];
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
            if (bits && t == seg * gx && tid == 0) flag(status, bits);   // once, by the segment's first task
            seg_ok = bits == 0;
            cur_seg = seg;
            si.stream = stream;
            si.po = po;
            si.pb = pb;
            si.nch = nch;
            si.spc = C / kSub;
            have_cur = have_next_raw = false;
            const uint32_t g0f = first_sub(t);
            have_first = seg_ok && g0f < a.blocks_per_seg;
            if (have_first) first_raw = issue_index(a, si, g0f + lane);
#pragma unroll
            for (int k = 0; k < kTabPer; ++k) {
                if (CODEC != EC_CODEC_EXP_GOLOMB && tid + k * kThreads < kTableVec) sm.h.tabv[tid + k * kThreads] = tv[k];
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
        if (!seg_ok) continue;   // uniform over the workgroup

        const uint32_t g0 = first_sub(t);   // the wave's first sub-chunk
        // the wave's next task, if it is in the same stream
        const uint32_t t1 = t + gridDim.x;
        const bool next_same = t1 < n_iter && seg_of(t1) == seg;
        const uint32_t g0n = first_sub(t1);
        const bool next_busy = next_same && g0n < a.blocks_per_seg;
        if (g0 >= a.blocks_per_seg) {   // uniform over the wave
            have_cur = have_next_raw = false;
            continue;
        }
        if (!have_cur) {   // nothing prefetched: this task's index and first blocks now
            cur = resolve(a, si, have_first ? first_raw : issue_index(a, si, g0 + lane), g0 + lane, status);
            issue_blocks<kStage>(si, cur, pre);
        }
        have_first = false;
        if (next_busy && !have_next_raw) next_raw = issue_index(a, si, g0n + lane);
        const LaneTask L = cur;
        const bool live = L.ok && L.cnt > 0;   // L.nv == 0 then means a sub-chunk without bits: corrupt
        // a whole run decoded from the lane's column: for two stages of at
        // most kStage blocks each; else when the wave's longest sub-chunk fits
        uint32_t nv_max = 0;
        if constexpr (!kTwo) {
            nv_max = L.nv;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) nv_max = max(nv_max, (uint32_t)__shfl_xor((int)nv_max, d, 64));
        }
        const bool fits = kTwo || 1 + 4 * nv_max <= kRows;   // uniform over the wave
        bool full = live && fits && L.cnt == kSub && L.nv > 0 && (!kTwo || L.nv <= (uint32_t)(2 * kStage));

        // stage 1 (two stages: the first kStage blocks), from registers
        if (fits) {
            static_for<0, kStage>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                if ((uint32_t)k < L.nv) {
                    lds_u32 *w = my_col + (1 + 4 * k) * 64;   // rows 1 + 4 k ...
                    w[0] = pre[k].x;
                    w[64] = pre[k].y;
                    w[128] = pre[k].z;
                    w[192] = pre[k].w;
                }
            });
            if (!kTwo && nv_max > (uint32_t)kStage)
                stage_rest(region + kRowBytes + 4 * lane, reinterpret_cast<const uint4 *>(si.stream + si.po) + L.blk0,
                           L.nv, kStage, nv_max);
        }
        // each lane reads only its own column: program order suffices
        asm volatile("" ::: "memory");
        auto prefetch_next = [&]() __attribute__((always_inline)) {
            // the next task's first blocks, and the index entries of the one after
            if (next_busy) {
                cur = resolve(a, si, next_raw, g0n + lane, status);
                issue_blocks<kStage>(si, cur, pre);
                have_cur = true;
                const uint32_t t2 = t1 + gridDim.x;
                const uint32_t g0nn = first_sub(t2);
                have_next_raw = t2 < n_iter && seg_of(t2) == seg && g0nn < a.blocks_per_seg;
                if (have_next_raw) next_raw = issue_index(a, si, g0nn + lane);
            } else {
                have_cur = have_next_raw = false;
            }
        };
        if constexpr (kTwo) {
            // the blocks after stage 1, in flight during the first half
            if (__ballot(full && L.nv > (uint32_t)kStage)) issue_blocks<kStage, kStage>(si, L, pre);
        } else {
            prefetch_next();
        }

        uint8_t *dst = a.out + (uint64_t)seg * a.out_stride + L.first_sym;
        const uint32_t ylim = region / 8 + kRows * 32 - 1;
        constexpr int kFull = CODEC == EC_CODEC_QLC ? 1 : 2;
        const uint32_t want = (uint32_t)(L.eb - L.blk0 * 128);
        ColBits S;
        S.col = 4 * lane;
        S.base = region / 8 + 31;
        S.Y = S.base + (uint32_t)(L.sb - L.blk0 * 128);
        S.ylim = ylim;
        uint32_t bad = 0;
        if (full)
            bad = decode_run<CODEC, PAIRS, kFull, ColBits, kTwo ? 0 : 2>(S, kSub, dst, l1, symtab, sm.h.deep,
                                                                        seg_max_len, seg_lens, seg_k_eg);

        uint32_t bh = 0;
        if constexpr (kTwo) {
            // stage 2: blocks bh .. nv - 1, where bh holds the first bit not
            // yet consumed.  The first half was read from stage 1 when no bit
            // before the position lay past it.
            const uint32_t pos = S.bit();
            bh = pos >> 7;
            full = full && pos <= (uint32_t)kStage * 128 && bh < L.nv && L.nv - bh <= (uint32_t)kStage;
            if (full) {
                // blocks bh .. kStage - 1 move down to slots 0 .. (slot j is
                // read before any later write lands on it: bh + j >= j)
                const uint32_t keep = min(L.nv, (uint32_t)kStage) - bh;   // bh <= kStage (pos bound)
#pragma nounroll
                for (uint32_t j = 0; j < keep; ++j) {
                    const lds_u32 *r = my_col + (1 + 4 * (bh + j)) * 64;
                    const uint32_t x0 = r[0], x1 = r[64], x2 = r[128], x3 = r[192];
                    lds_u32 *w = my_col + (1 + 4 * j) * 64;
                    w[0] = x0;
                    w[64] = x1;
                    w[128] = x2;
                    w[192] = x3;
                }
                // block kStage + k goes to slot keep + k (at most kStage - 1)
                static_for<0, kStage>([&](auto kc) __attribute__((always_inline)) {
                    constexpr int k = decltype(kc)::value;
                    if ((uint32_t)(kStage + k) < L.nv) {
                        lds_u32 *w = my_col + (1 + 4 * (keep + k)) * 64;
                        w[0] = pre[k].x;
                        w[64] = pre[k].y;
                        w[128] = pre[k].z;
                        w[192] = pre[k].w;
                    }
                });
                S.Y -= bh * 128;
            } else {
                bh = 0;
            }
            asm volatile("" ::: "memory");
            prefetch_next();
        }

        bool corrupt = false;
        if (full) {
            if constexpr (kTwo)
                bad |= decode_run<CODEC, PAIRS, kFull, ColBits, 1>(S, kSub, dst, l1, symtab, sm.h.deep, seg_max_len,
                                                                   seg_lens, seg_k_eg);
            corrupt = (bad & ~0xffu) || S.bit() + bh * 128 != want;
        }
        // the zero padding after a chunk's last sub-chunk
        const bool pad_check = full && !corrupt && L.pad_end > L.eb;
        if (__ballot(pad_check))
            if (pad_check) corrupt = padding_set(reinterpret_cast<const uint32_t *>(si.stream + si.po), L.eb, L.pad_end);
        if (__ballot(live && !full))
            if (live && !full)
                decode_rest<CODEC, PAIRS>(L, reinterpret_cast<const uint32_t *>(si.stream + si.po), si.pb, dst, l1,
                                          symtab, sm.h.deep, seg_max_len, seg_lens, seg_k_eg, status);
        if (corrupt) flag(status, EC_S_CORRUPT);
        // the column is rewritten at the next task, after this lane's reads
        asm volatile("" ::: "memory");
    }
}

// Workgroups of a persistent launch: as many as can be resident at once,
// never more than there are tasks.
template <class K>
hipError_t decode_grid(K kernel, uint32_t threads, uint32_t n_tasks, uint32_t *grid) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    if (e != hipSuccess) return e;
    const uint64_t g = (uint64_t)(per_cu > 0 ? per_cu : 1) * (uint64_t)(cus > 0 ? cus : 1);
    *grid = g < n_tasks ? (uint32_t)g : n_tasks;
    return hipSuccess;
}

template <int CODEC, int PAIRS>
hipError_t launch_one(const DecodeArgs &a, hipStream_t s) {
    constexpr uint32_t kThreads = 64 * waves_for<CODEC>();
    uint32_t gx = (a.blocks_per_seg + kThreads - 1) / kThreads;
    if (gx == 0) gx = 1;   // still validate the header
    // one stream: up to one workgroup per run of 64 sub-chunks, its waves
    // spread over the workgroups; else up to one per task
    const uint32_t runs = (a.blocks_per_seg + 63) / 64;
    const uint32_t cap = a.n_seg == 1 ? (runs > gx ? runs : gx) : gx * a.n_seg;
    uint32_t grid = 0;
    const hipError_t e = decode_grid(decode_kernel<CODEC, PAIRS>, kThreads, cap, &grid);
    if (e != hipSuccess) return e;
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
