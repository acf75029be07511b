// Chunk-parallel decoder.
//
// Every 256-symbol sub-chunk starts at a bit offset recorded in the stream
// index, so one lane decodes one sub-chunk serially and a wave64 decodes 64
// consecutive sub-chunks side by side.  Their compressed bits form one
// contiguous span of the payload (about 14 KiB at 16384-symbol chunks), which
// the wave first copies into its own LDS region (16 KiB, 15 KiB for Huffman)
// with coalesced 16-byte loads.
// The decode loop then reads only LDS: a 32-bit window at any bit position is
// one two-word LDS read plus a funnel shift and serves two codes of up to 16
// bits each.  (A global load inside the loop would stall on the output
// stores too: one counter tracks both.)  A span larger than the LDS region
// (data that barely compresses) is decoded straight from global memory.
//   QLC      the 3-bit prefix gives the code length through a packed constant
//            (no memory access on the dependency chain); the top 11 bits index
//            a 2048-entry LDS table that yields the byte or flags an unused
//            suffix.
//   Huffman  the top 13 bits index a 16 KiB LDS table that yields the byte
//            and the length of every code of up to 13 bits; longer codes
//            (rare) are found by comparing a 40-bit window against the
//            canonical code limits.
//   EG       count leading zeros z; the code is 2z + k + 1 bits; rank -> byte
//            through a 256-entry LDS table.
// After its last symbol a lane checks that it stopped exactly where the index
// says its sub-chunk ends.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kGuardBytes = 1536;               // > 256 codes x 40 bits of overrun

// Bits of a lane's sub-chunk staged in LDS.  The wave's span is copied to
// words 4.. of its region (words 0-3 are zero, word 3 is the guard before
// the span).  x is the absolute LDS bit address of the guard word's start
// plus 31 plus the span bit position, so the word holding the bit before the
// read position is x >> 5 and a 32-bit window never needs a special case.
// Positions only move forward from a validated start by at most 40 bits a
// code, and the region is followed by guard words, so reads stay inside the
// allocation even for corrupt streams.
struct SpanBits {
    static constexpr bool kStaged = true;
    uint32_t x;      // absolute LDS bit address of the position, plus 31
    uint32_t base;   // absolute LDS bit address of the span's first bit

    typedef __attribute__((address_space(3))) const uint32_t lds_word;
    __device__ __forceinline__ uint32_t at(uint32_t xx) const {
        // word address from the bit address by a shift and a mask (no base
        // to add); the two words hold the bit before the position and the
        // 31 bits after it
        lds_word *w = (lds_word *)(size_t)((xx >> 3) & ~3u);
        return __builtin_amdgcn_alignbit(w[0], w[1], ~xx);
    }
    __device__ __forceinline__ uint32_t win() const { return at(x); }
    __device__ __forceinline__ uint64_t win64() const { return ((uint64_t)at(x) << 32) | at(x + 32u); }
    __device__ __forceinline__ void adv(uint32_t l) { x += l; }
    __device__ __forceinline__ void prepare() {}
    __device__ __forceinline__ uint64_t bit() const { return x + 1u - base; }   // span-relative position
};

// Bits of a lane's sub-chunk read straight from global memory (spans that
// do not fit in LDS): a 64-bit MSB-aligned buffer refilled 32 bits at a time,
// loads clamped to the payload.
struct GlobalBits {
    static constexpr bool kStaged = false;
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
// 40-bit left-justified window.  Returns symbol | length << 8.
__device__ __noinline__ uint32_t huff_deep(uint64_t window, const DeepTables *dt, const uint8_t *sym, uint32_t mx) {
    const uint64_t w40 = window >> (64 - EC_MAX_CODE_LEN);
    uint32_t l = kHuffBits + 1;
    while (l < mx && w40 >= dt->limit[l - kHuffBits - 1]) ++l;
    const uint32_t i = l - kHuffBits - 1;
    const uint64_t code = w40 >> (EC_MAX_CODE_LEN - l);
    const uint32_t idx = dt->first_idx[i] + (uint32_t)(code - dt->first_code[i]);
    return sym[idx & 255] | (l << 8);
}

// Decode one 256-symbol run (or the cnt < 256 symbols of a segment's last
// run) from source S into dst; returns the bits of the QLC / EG "not a
// codeword" flags (bit 8 and up).
template <int CODEC, int PAIRS, class Src>
__device__ __forceinline__ uint32_t decode_run(Src &S, uint32_t cnt, uint8_t *dst, const uint16_t *l1,
                                               const uint8_t *symtab, const DeepTables *dt, uint32_t max_len,
                                               uint32_t lens, uint32_t k_eg) {
    uint32_t bad = 0;
    // The code that starts window w: its table entry (symbol in byte 0; for
    // QLC bit 8 flags an unused suffix) and its length.  QLC takes the length
    // from the 3-bit prefix through the packed constant, off the memory
    // dependency chain; Huffman and EG entries carry it in bits 8 and up.
    struct Code {
        uint32_t e, len;
    };
    auto code_at = [&](uint32_t w) __attribute__((always_inline)) -> Code {
        if (CODEC == EC_CODEC_QLC) {
            return Code{l1[w >> 21], (lens >> ((w >> 29) << 2)) & 15u};
        } else if (CODEC == EC_CODEC_HUFFMAN) {
            uint32_t e = l1[w >> (32 - kHuffBits)];
            if (e < 256u) e = huff_deep(S.win64(), dt, symtab, max_len);
            return Code{e, e >> 8};
        } else {
            const uint32_t zr = __clz(w);
            const uint32_t z = zr < 8u ? zr : 8u;   // more zeros: not a codeword
            const uint32_t l = 2 * z + k_eg + 1;
            const uint32_t rank = (w >> (32 - l)) - (1u << k_eg);
            bad |= rank | (zr > 8u ? kQlcInvalid : 0u);
            return Code{symtab[rank & 255u], l};
        }
    };
    auto one = [&]() __attribute__((always_inline)) -> uint32_t {
        const Code c = code_at(S.win());
        if (CODEC == EC_CODEC_QLC) bad |= c.e;
        S.adv(c.len);
        return c.e & 0xffu;
    };
    // two codes from one window when both fit in it; returns byte0 | byte1 << 8
    auto two = [&]() __attribute__((always_inline)) -> uint32_t {
        const uint32_t w = S.win();
        const Code c1 = code_at(w);
        Code c2;
        if (CODEC == EC_CODEC_HUFFMAN) {
            // the second code's table index comes from the same window when
            // the first code left at least 13 bits of it
            S.adv(c1.len);
            const uint32_t w2 = c1.len <= 32u - kHuffBits ? w << c1.len : S.win();
            c2.e = l1[w2 >> (32 - kHuffBits)];
            if (c2.e < 256u) c2.e = huff_deep(S.win64(), dt, symtab, max_len);
            S.adv(c2.e >> 8);
        } else {
            c2 = code_at(w << c1.len);
            S.adv(c1.len + c2.len);
            if (CODEC == EC_CODEC_QLC) bad |= c1.e | c2.e;
        }
        return __builtin_amdgcn_perm(c2.e, c1.e, 0x0c0c0400u);   // byte 0 of c1.e, byte 0 of c2.e
    };
    // eight codes -> two output words
    auto eight = [&](uint32_t &lo, uint32_t &hi) __attribute__((always_inline)) {
        S.prepare();
        if (PAIRS) {
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

    if (cnt == kSub && Src::kStaged) {
        // 128 decoded bytes are collected in registers and written as one
        // whole cache line: 16-byte stores to 64 lanes' separate lines leave
        // partial lines in L2 that get written back more than once
        for (int half = 0; half < 2; ++half) {
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
        }
    } else if (cnt == kSub) {
        for (int i = 0; i < kSub / 16; ++i) {
            uint32_t o[4];
            eight(o[0], o[1]);
            eight(o[2], o[3]);
            *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else {
        for (uint32_t k = 0; k < cnt; ++k) dst[k] = (uint8_t)one();
    }
    return bad;
}

// Index entries of one lane's sub-chunk and of its wave's span, as loaded
// from the stream (resolved later, so that the loads can be in flight while
// the wave decodes an earlier task).
struct IndexRaw {
    uint64_t co0, co1;        // the lane's chunk: byte offsets of its start and end in the payload
    uint64_t slo, shi;        // the wave's span: first chunk's start, last chunk's end
    uint32_t e_start, e_end;  // the lane's sub-chunk: start and end bit in its chunk
};

// A wave's task: 64 consecutive sub-chunks of one stream, one per lane.
struct Plan {
    uint64_t co0, span_lo;
    uint32_t e_start, e_end, cnt, nblk;
    uint64_t first_sym;
    bool active, ok, fits;
};

// Stream fields the tasks of a segment share (validated once per segment).
struct StreamInfo {
    const uint8_t *stream;
    uint64_t po, pb;
    uint32_t nch, spc;
};

__device__ __forceinline__ IndexRaw issue_index(const DecodeArgs &a, const StreamInfo &si, uint32_t g0,
                                                uint32_t lane) {
    const uint64_t *chunk_off = reinterpret_cast<const uint64_t *>(si.stream + kHeaderBytes);
    const uint32_t *sub_end = reinterpret_cast<const uint32_t *>(si.stream + kHeaderBytes + 8ull * (si.nch + 1));
    const uint32_t g = g0 + lane;
    const uint32_t gl = g < a.blocks_per_seg ? g : a.blocks_per_seg - 1;
    const uint32_t c = gl / si.spc, j = gl - c * si.spc;
    const uint32_t g_last = g0 + 63 < a.blocks_per_seg ? g0 + 63 : a.blocks_per_seg - 1;
    IndexRaw r;
    r.co0 = chunk_off[c];
    r.co1 = chunk_off[c + 1];
    r.e_end = sub_end[(uint64_t)c * si.spc + j];
    r.e_start = j ? sub_end[(uint64_t)c * si.spc + j - 1] : 0u;
    r.slo = chunk_off[g0 / si.spc];
    r.shi = chunk_off[g_last / si.spc + 1];
    return r;
}

// Checks the lane's index entries (flags a corrupt index) and decides
// whether the wave's span fits its LDS region.
template <uint32_t kSpan>
__device__ __forceinline__ Plan resolve(const DecodeArgs &a, const StreamInfo &si, const IndexRaw &r, uint32_t g0,
                                        uint32_t lane, uint32_t *status) {
    Plan p;
    const uint32_t g = g0 + lane;
    p.active = g < a.blocks_per_seg;
    p.ok = p.active && r.co0 <= r.co1 && r.co1 <= si.pb && !(r.co0 & 15) &&
           (uint64_t)r.e_end <= (r.co1 - r.co0) * 8 && r.e_start <= r.e_end;
    if (p.active && !p.ok) or_status(status, EC_S_CORRUPT);
    p.span_lo = r.slo & ~15ull;
    const uint64_t span_hi = r.shi;
    bool fits = p.span_lo <= span_hi && span_hi <= si.pb && span_hi - p.span_lo <= kSpan;
    p.fits = fits && __ballot(p.ok && (r.co0 < p.span_lo || r.co1 > span_hi)) == 0;
    p.nblk = p.fits ? (uint32_t)((span_hi - p.span_lo + 15) >> 4) : 0u;
    p.co0 = r.co0;
    p.e_start = r.e_start;
    p.e_end = r.e_end;
    p.first_sym = (uint64_t)g * kSub;
    p.cnt = !p.active ? 0u : (a.seg_n - p.first_sym < kSub ? (uint32_t)(a.seg_n - p.first_sym) : (uint32_t)kSub);
    return p;
}

// The wave's span as 16-byte blocks, lane + 64 k, loaded into registers
// (indexes clamped to the span, so every load stays inside it).
template <int K>
__device__ __forceinline__ void issue_span(const StreamInfo &si, const Plan &p, uint32_t lane, uint4 (&v)[K]) {
    if (!p.fits || p.nblk == 0) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(si.stream + si.po) + (p.span_lo >> 4);
    const uint32_t last = p.nblk - 1;
    static_for<0, K>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        v[k] = src[min(lane + 64u * k, last)];
    });
}

// Persistent workgroups: workgroup b takes tasks b, b + G, ... (G = grid);
// a task is 256 consecutive sub-chunks of one stream, 64 per wave.  For QLC
// the index entries of the wave's task after next and the compressed span of
// its next task are loaded while it decodes the current one.
template <int CODEC, int PAIRS>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeArgs a) {
    // Staging per wave: 16 KiB, or 15 KiB next to the 16 KiB Huffman table,
    // so that two workgroups still fit in a CU's 160 KiB of LDS.
    constexpr uint32_t kSpan = CODEC == EC_CODEC_HUFFMAN ? 15360 : 16384;
    constexpr int kSpanVec = kSpan / 16 / 64;   // 16-byte blocks per lane
    // Keeping the next span in registers costs 64 VGPRs: QLC's decode loop
    // has them to spare, the Huffman and EG loops do not.
    constexpr bool kPrefetch = CODEC == EC_CODEC_QLC;
    constexpr uint32_t kTableVec = CODEC == EC_CODEC_QLC       ? kL1Size * 2 / 16
                                   : CODEC == EC_CODEC_HUFFMAN ? kHuffSize * 2 / 16
                                                               : 1;
    // tables first, so that their addresses fit the LDS instructions' offset field
    struct Smem {
        uint4 tabv[kTableVec];
        uint8_t symtab[256];       // EG: rank -> byte; Huffman: canonical order -> byte
        DeepTables deep[1];        // Huffman only
        uint64_t po, pb;
        uint32_t ok, nch, spc;
        uint32_t pad_;
        uint4 spans[kWaves][(kSpan + 32) / 16];
        uint4 guard[kGuardBytes / 16];
    };
    __shared__ Smem sm;
    const uint16_t *l1 = reinterpret_cast<const uint16_t *>(sm.tabv);
    uint8_t *symtab = sm.symtab;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t gx = (a.blocks_per_seg + kThreads - 1) / kThreads > 0 ? (a.blocks_per_seg + kThreads - 1) / kThreads
                                                                           : 1u;
    const uint32_t n_tasks = gx * a.n_seg;
    uint4 *region = sm.spans[wave];
    // word 3 of the region is the guard word right before the span
    const uint32_t region_base = (uint32_t)(size_t)(__attribute__((address_space(3))) const uint4 *)region * 8 + 4 * 32;

    uint32_t cur_seg = ~0u;
    StreamInfo si = {};
    const DevTables *tab = nullptr;
    uint32_t *status = nullptr;
    bool have_cur = false, have_next_raw = false;
    Plan cur = {};
    IndexRaw next_raw = {};
    uint4 span_regs[kPrefetch ? kSpanVec : 1];
#pragma unroll
    for (int k = 0; k < (kPrefetch ? kSpanVec : 1); ++k) span_regs[k] = make_uint4(0, 0, 0, 0);

    for (uint32_t t = blockIdx.x; t < n_tasks; t += gridDim.x) {
        const uint32_t seg = t / gx, bx = t - seg * gx;
        if (seg != cur_seg) {
            __syncthreads();   // the previous segment's tables are no longer read
            tab = seg_tables<DecodeArgs>(seg);
            if (CODEC == EC_CODEC_QLC) sm.tabv[tid] = reinterpret_cast<const uint4 *>(tab->l1)[tid];
            if (CODEC == EC_CODEC_HUFFMAN) {
#pragma unroll
                for (int k = 0; k < (int)kTableVec / kThreads; ++k)
                    sm.tabv[tid + k * kThreads] = reinterpret_cast<const uint4 *>(tab->hl1)[tid + k * kThreads];
            }
            if (CODEC != EC_CODEC_QLC) symtab[tid] = tab->sym[tid];
            if constexpr (CODEC == EC_CODEC_HUFFMAN) {
                constexpr uint32_t kDeep = EC_MAX_CODE_LEN - kHuffBits;
                if (tid < kDeep) {
                    sm.deep[0].limit[tid] = tab->limit[kHuffBits + 1 + tid];
                    sm.deep[0].first_code[tid] = tab->first_code[kHuffBits + 1 + tid];
                    sm.deep[0].first_idx[tid] = tab->first_idx[kHuffBits + 1 + tid];
                }
            }
            const uint8_t *stream = a.in + (uint64_t)seg * a.in_stride;
            status = a.status ? a.status + seg : nullptr;
            if (tid == 0) {
                const uint64_t *h = reinterpret_cast<const uint64_t *>(stream);
                const uint64_t h0 = h[0], n = h[1], h2 = h[2], po = h[3], pb = h[4], id = h[5];
                const uint32_t magic = (uint32_t)h0, version = (uint32_t)(h0 >> 32) & 0xffffu;
                const uint32_t codec = (uint32_t)(h0 >> 48) & 0xffu, flags = (uint32_t)(h0 >> 56);
                const uint32_t C = (uint32_t)h2, nch = (uint32_t)(h2 >> 32);
                uint32_t bits = 0;
                if (magic != kMagic || version != kVersion || (flags & ~1u)) {
                    bits = EC_S_BAD_HEADER;
                } else if (codec != tab->codec || id != tab->codebook_id) {
                    bits = EC_S_CODEBOOK_MISMATCH;
                } else if (n != a.seg_n || C == 0 || (C % kSub) || C > kMaxChunk ||
                           (uint64_t)nch != (n + C - 1) / C) {
                    bits = EC_S_BAD_HEADER;
                } else {
                    uint64_t end =
                        kHeaderBytes + 8ull * (nch + 1) + 4ull * nch * (C / kSub) + ((flags & 1) ? 256 : 0);
                    end = (end + 255) / 256 * 256;
                    if (po != end || pb % 16 || po + pb > a.in_len || (n > 0 && pb == 0) || pb >= (1ull << 36))
                        bits = EC_S_BAD_HEADER;
                }
                sm.ok = bits == 0;
                if (bits && bx == 0) or_status(status, bits);
                sm.nch = nch;
                sm.spc = C / kSub;
                sm.po = po;
                sm.pb = pb;
            }
            __syncthreads();
            cur_seg = seg;
            si.stream = stream;
            si.po = sm.po;
            si.pb = sm.pb;
            si.nch = sm.nch;
            si.spc = sm.spc;
            have_cur = have_next_raw = false;
        }
        if (!sm.ok) continue;   // uniform over the workgroup

        const uint32_t g0 = bx * kThreads + wave * 64;   // the wave's first sub-chunk
        const bool wave_busy = g0 < a.blocks_per_seg;
        // the wave's next task, if it is in the same stream
        const uint32_t t1 = t + gridDim.x;
        const bool next_same = t1 < n_tasks && t1 / gx == seg;
        const uint32_t g0n = (t1 - seg * gx) * kThreads + wave * 64;
        const bool next_busy = next_same && g0n < a.blocks_per_seg;

        if (wave_busy) {
            if (!have_cur) {   // nothing prefetched: load this task's index and span now
                const IndexRaw r = issue_index(a, si, g0, lane);
                cur = resolve<kSpan>(a, si, r, g0, lane, status);
                if constexpr (kPrefetch) issue_span<kSpanVec>(si, cur, lane, span_regs);
            }
            if (kPrefetch && next_busy && !have_next_raw) next_raw = issue_index(a, si, g0n, lane);
            // stage the span: region block 0 is zero (its last word is the
            // guard before the span), the span follows from block 1, and a
            // zero block closes it
            if (cur.fits) {
                if constexpr (kPrefetch) {
                    static_for<0, kSpanVec>([&](auto kc) __attribute__((always_inline)) {
                        constexpr int k = decltype(kc)::value;
                        if (lane + 64u * k < cur.nblk) region[1 + lane + 64 * k] = span_regs[k];
                    });
                } else {
                    // coalesced copy, four 1 KiB loads in flight per pass
                    const uint4 *src = reinterpret_cast<const uint4 *>(si.stream + si.po) + (cur.span_lo >> 4);
                    const uint32_t nblk = cur.nblk;
                    for (uint32_t i = lane; i < nblk; i += 256) {
                        const uint32_t last = nblk - 1;
                        const uint4 v0 = src[min(i, last)], v1 = src[min(i + 64, last)];
                        const uint4 v2 = src[min(i + 128, last)], v3 = src[min(i + 192, last)];
                        region[1 + i] = v0;
                        if (i + 64 < nblk) region[1 + i + 64] = v1;
                        if (i + 128 < nblk) region[1 + i + 128] = v2;
                        if (i + 192 < nblk) region[1 + i + 192] = v3;
                    }
                }
                if (lane == 0) region[0] = make_uint4(0u, 0u, 0u, 0u);
                if (lane == 1) region[1 + cur.nblk] = make_uint4(0u, 0u, 0u, 0u);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const Plan p = cur;
            // prefetch: the next task's span, and the index entries of the one after
            if (kPrefetch && next_busy) {
                cur = resolve<kSpan>(a, si, next_raw, g0n, lane, status);
                if constexpr (kPrefetch) issue_span<kSpanVec>(si, cur, lane, span_regs);
                have_cur = true;
                const uint32_t t2 = t1 + gridDim.x;
                const uint32_t g0nn = (t2 - seg * gx) * kThreads + wave * 64;
                have_next_raw = t2 < n_tasks && t2 / gx == seg && g0nn < a.blocks_per_seg;
                if (have_next_raw) next_raw = issue_index(a, si, g0nn, lane);
            } else {
                have_cur = have_next_raw = false;
            }

            uint8_t *dst = a.out + (uint64_t)seg * a.out_stride + p.first_sym;
            const uint32_t lens = tab->qlc_lens;
            const uint32_t k_eg = (uint32_t)tab->eg_k;
            uint32_t bad = 0;
            uint64_t end_pos = 0, want_pos = 0;
            if (p.fits) {
                if (p.ok) {
                    SpanBits S;
                    S.base = region_base;
                    S.x = S.base + (uint32_t)((p.co0 - p.span_lo) * 8 + p.e_start) - 1u;
                    bad = decode_run<CODEC, PAIRS>(S, p.cnt, dst, l1, symtab, sm.deep, tab->max_len, lens, k_eg);
                    end_pos = S.bit();
                    want_pos = (p.co0 - p.span_lo) * 8 + p.e_end;
                }
            } else if (p.ok) {
                GlobalBits S;
                S.init(reinterpret_cast<const uint32_t *>(si.stream + si.po), si.pb >> 2, p.co0 * 8 + p.e_start);
                bad = decode_run<CODEC, PAIRS>(S, p.cnt, dst, l1, symtab, sm.deep, tab->max_len, lens, k_eg);
                end_pos = S.bit();
                want_pos = p.co0 * 8 + p.e_end;
            }
            if (p.ok && ((bad & ~0xffu) || end_pos != want_pos)) or_status(status, EC_S_CORRUPT);
            // the region is rewritten at the next task: all lanes' reads first
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else {
            have_cur = have_next_raw = false;
        }
    }
}

// Workgroups of a persistent launch: as many as can be resident at once,
// never more than there are tasks.
template <class K>
hipError_t decode_grid(K kernel, uint32_t n_tasks, uint32_t *grid) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0);
    if (e != hipSuccess) return e;
    const uint64_t g = (uint64_t)(per_cu > 0 ? per_cu : 1) * (uint64_t)(cus > 0 ? cus : 1);
    *grid = g < n_tasks ? (uint32_t)g : n_tasks;
    return hipSuccess;
}

template <int CODEC, int PAIRS>
hipError_t launch_one(const DecodeArgs &a, hipStream_t s) {
    uint32_t gx = (a.blocks_per_seg + kThreads - 1) / kThreads;
    if (gx == 0) gx = 1;   // still validate the header
    uint32_t grid = 0;
    const hipError_t e = decode_grid(decode_kernel<CODEC, PAIRS>, gx * a.n_seg, &grid);
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
