// Chunked fixed-codebook encoder: three launches on the caller's stream.
//
//   1. encode_sizes_kernel (one workgroup of 256 threads per chunk): loads
//      the chunk as 16-byte pieces (piece q = r * 256 + thread, so each load
//      instruction of a wave reads 1 KiB of contiguous bytes), sums each
//      piece's code lengths from a byte table in LDS, scans the piece lengths
//      over the workgroup and writes the chunk's sub_end[] entries (end bit
//      of every 256-symbol sub-chunk) and its size in 16-byte units.
//   2. encode_offsets_kernel (one workgroup per stream): exclusive scan of
//      the stream's chunk sizes -> chunk_off[], payload_bytes and the stream
//      length; writes the header, the embedded code lengths and the zero
//      padding in front of the payload; flags a stream that does not fit.
//      Only for streams of more than kPlaceMaxChunks chunks: for shorter
//      ones the first pack launch does this itself (every workgroup sums the
//      sizes of the chunks before its own, the stream's last chunk writes
//      the header, its first chunk the index tail), one launch fewer.
//   3. encode_pack_*_kernel (one workgroup per chunk): loads the chunk again,
//      looks each symbol's code up in the codebook's LUT in LDS (code
//      left-aligned, length in the low byte), scans the piece lengths, ORs the
//      codes into a zeroed LDS bit buffer (MSB first) and stores the finished
//      chunk at its offset with coalesced stores.
// Every chunk knows its place before it is packed, so no workgroup ever
// waits on another one: the launches need no co-residency, tickets or
// spinning, at the price of reading the input twice.  When the sizes come
// from the caller (made by the histogram's pass over the same input, see
// histogram.hip), launch 1 is skipped: the packer writes the sub_end[]
// entries and checks its chunk's size against the one it was given, and the
// input is read once by the encode.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kPiece = 16;                     // symbols per piece (one 16-byte load)
constexpr int kRowSyms = kThreads * kPiece;    // 4096

// Byte K (compile-time) of a 16-byte piece, in memory order.
template <int K>
__device__ __forceinline__ uint32_t byte_k(const uint4 &v) {
    constexpr int w = K >> 2, sh = 8 * (K & 3);
    const uint32_t x = w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
    return (x >> sh) & 0xffu;
}

// Where chunk t of the launch lives.
struct ChunkPos {
    uint32_t seg, lc, cn;
    const uint8_t *src;
    uint8_t *out;
};

__device__ __forceinline__ ChunkPos chunk_pos(const EncodeArgs &a, uint32_t t) {
    ChunkPos p;
    p.seg = t / a.chunks_per_seg;
    p.lc = t - p.seg * a.chunks_per_seg;
    const uint64_t first = (uint64_t)p.lc * a.chunk_symbols;
    const uint64_t left = a.seg_n - first;
    p.cn = left < a.chunk_symbols ? (uint32_t)left : a.chunk_symbols;
    p.src = a.in + (uint64_t)p.seg * a.in_stride + first;
    p.out = a.out + (uint64_t)p.seg * a.out_stride;
    return p;
}

// Load the chunk's pieces: piece q = r * 256 + tid, vb[r] valid bytes.  A
// piece holding the segment's last byte is read as its whole 16-byte block
// (the input is 16-byte aligned, so the block never crosses a page); bytes
// past the end are ignored through vb.  Pieces past the end read nothing.
template <int ROWS>
__device__ __forceinline__ void load_pieces(const uint8_t *src, uint32_t cn, uint32_t tid, uint4 (&v)[ROWS],
                                            uint32_t (&vb)[ROWS]) {
    if (cn == (uint32_t)(ROWS * kRowSyms)) {   // whole chunk present: plain loads
        static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            vb[r] = kPiece;
            v[r] = *reinterpret_cast<const uint4 *>(src + (uint32_t)(r * kThreads + tid) * kPiece);
        });
        return;
    }
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        const uint32_t off = (uint32_t)(r * kThreads + tid) * kPiece;
        vb[r] = off < cn ? min(cn - off, (uint32_t)kPiece) : 0u;
        v[r] = make_uint4(0, 0, 0, 0);
        if (off < cn) v[r] = *reinterpret_cast<const uint4 *>(src + off);
    });
}

// Scan of piece lengths over the workgroup: per row a wave-inclusive scan,
// then the four waves' totals through LDS.  Gives every piece's exclusive
// bit offset in the chunk, the rows' starts and lengths, and the chunk total.
template <int ROWS>
__device__ __forceinline__ uint32_t scan_pieces(const uint32_t (&plen)[ROWS], uint32_t lane, uint32_t wave,
                                                uint32_t (*wave_tot)[kThreads / 64], uint32_t (&excl)[ROWS],
                                                uint32_t (&row_start)[ROWS], uint32_t (&row_bits)[ROWS]) {
    uint32_t incl[ROWS];
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        const uint32_t x = wave_incl_scan(plen[r]);
        incl[r] = x;
        if (lane == 63) wave_tot[r][wave] = x;
    });
    __syncthreads();
    uint32_t total = 0;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        uint32_t before = 0, rt = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            const uint32_t t = wave_tot[r][w];
            before += (uint32_t)w < wave ? t : 0u;
            rt += t;
        }
        row_start[r] = total;
        row_bits[r] = rt;
        excl[r] = total + before + incl[r] - plen[r];
        total += rt;
    });
    return total;
}

// ---------------------------------------------------------------- 1. sizes

// sub_end[]: the end bit of every 256-symbol sub-chunk, written by the
// thread holding the sub-chunk's last piece
template <int ROWS>
__device__ __forceinline__ void write_sub_end(const EncodeArgs &a, const ChunkPos &p, uint32_t tid,
                                              const uint32_t (&excl)[ROWS], const uint32_t (&plen)[ROWS]) {
    const uint32_t spc = a.chunk_symbols / kSub;
    uint32_t *sub_end = reinterpret_cast<uint32_t *>(p.out + a.sub_at) + (uint64_t)p.lc * spc;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        const uint32_t q = (uint32_t)r * kThreads + tid;
        if ((tid & 15) == 15 && q < a.chunk_symbols / kPiece) sub_end[q >> 4] = excl[r] + plen[r];
    });
}

template <int ROWS>
__global__ __launch_bounds__(kThreads) void encode_sizes_kernel(const EncodeArgs a) {
    __shared__ uint8_t len8[256];
    __shared__ uint32_t wave_tot[ROWS][kThreads / 64];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const ChunkPos p = chunk_pos(a, blockIdx.x);
    uint4 v[ROWS];
    uint32_t vb[ROWS];
    load_pieces<ROWS>(p.src, p.cn, tid, v, vb);
    len8[tid] = seg_tables<EncodeArgs>(p.seg)->code_len[tid];
    __syncthreads();

    uint32_t plen[ROWS];
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        uint32_t x = 0;
        if (vb[r] == kPiece) {
            static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
                x += len8[byte_k<decltype(kc)::value>(v[r])];
            });
        } else {
            static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                x += (uint32_t)k < vb[r] ? (uint32_t)len8[byte_k<k>(v[r])] : 0u;
            });
        }
        plen[r] = x;
    });
    uint32_t excl[ROWS], row_start[ROWS], row_bits[ROWS];
    const uint32_t chunk_bits = scan_pieces<ROWS>(plen, lane, wave, wave_tot, excl, row_start, row_bits);
    write_sub_end<ROWS>(a, p, tid, excl, plen);
    if (tid == 0) a.sizes[blockIdx.x] = (chunk_bits + 127) >> 7;
}

// -------------------------------------------------------------- 2. offsets

constexpr int kScanThreads = 1024;

// Header fields, chunk_off[n_chunks] and the stream length of stream `seg`
// whose payload has `payload` bytes; flags a stream that does not fit and an
// unusable codebook.  One thread.
__device__ void write_header(const EncodeArgs &a, uint32_t seg, uint64_t payload) {
    const DevTables *tab = seg_tables<EncodeArgs>(seg);
    uint8_t *out = a.out + (uint64_t)seg * a.out_stride;
    const uint32_t n = a.chunks_per_seg;
    reinterpret_cast<uint64_t *>(out + kHeaderBytes)[n] = payload;
    const uint64_t end = (uint64_t)a.payload_offset + payload;
    uint64_t *h = reinterpret_cast<uint64_t *>(out);
    h[0] = (uint64_t)kMagic | ((uint64_t)kVersion << 32) | ((uint64_t)tab->codec << 48) |
           ((uint64_t)(a.embed_lengths ? 1 : 0) << 56);
    h[1] = a.seg_n;
    h[2] = (uint64_t)a.chunk_symbols | ((uint64_t)n << 32);
    h[3] = a.payload_offset;
    h[4] = payload;
    h[5] = tab->codebook_id;
    h[6] = 0;
    h[7] = 0;
    a.out_len[seg] = end;
    if (end > a.out_cap) or_status(a.status ? a.status + seg : nullptr, EC_S_CAPACITY);
    if (tab->codec == 0) or_status(a.status ? a.status + seg : nullptr, EC_S_BAD_CODEBOOK);
}

// The embedded code lengths and the zero fill from the end of the index to
// the payload of stream `seg`, by threads tid of nthreads.
__device__ void write_index_tail(const EncodeArgs &a, uint32_t seg, uint32_t tid, uint32_t nthreads) {
    const DevTables *tab = seg_tables<EncodeArgs>(seg);
    uint8_t *out = a.out + (uint64_t)seg * a.out_stride;
    const uint32_t index_end = a.sub_at + 4u * a.chunks_per_seg * (a.chunk_symbols / kSub);
    uint32_t pad_from = index_end;
    if (a.embed_lengths) {
        for (uint32_t i = tid; i < 256; i += nthreads) out[index_end + i] = tab->code_len[i];
        pad_from += 256;
    }
    for (uint32_t i = pad_from + tid; i < a.payload_offset; i += nthreads) out[i] = 0;
}

// chunk_off[], the header, the stream length, the embedded code lengths and
// the zero fill up to the payload of stream `blockIdx.x` (long streams).
__global__ __launch_bounds__(kScanThreads) void encode_offsets_kernel(const EncodeArgs a) {
    __shared__ uint64_t wsum[kScanThreads / 64];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t seg = blockIdx.x;
    uint8_t *out = a.out + (uint64_t)seg * a.out_stride;
    const uint32_t n = a.chunks_per_seg;
    const uint32_t *sz = a.sizes + (uint64_t)seg * n;
    uint64_t *chunk_off = reinterpret_cast<uint64_t *>(out + kHeaderBytes);

    // Each thread owns a run of consecutive chunks.  Up to four chunks a
    // thread (up to 4096 chunks a stream) come in one 16-byte load and stay
    // in registers; longer runs loop.
    const uint32_t per = (n + kScanThreads - 1) / kScanThreads;
    const uint32_t lo = min(n, tid * per), hi = min(n, lo + per);
    uint64_t mine = 0;
    uint32_t s4[4] = {0, 0, 0, 0};
    const bool quad = per <= 4;
    if (quad) {
        if (per == 4 && hi == lo + 4 && !((uintptr_t)(sz + lo) & 15)) {
            const uint4 v = *reinterpret_cast<const uint4 *>(sz + lo);
            s4[0] = v.x;
            s4[1] = v.y;
            s4[2] = v.z;
            s4[3] = v.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) s4[k] = lo + k < hi ? sz[lo + k] : 0u;
        }
        mine = (uint64_t)s4[0] + s4[1] + s4[2] + s4[3];
    } else {
        for (uint32_t i = lo; i < hi; ++i) mine += sz[i];
    }
    uint64_t x = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t y = __shfl_up(x, d, 64);
        if (lane >= (uint32_t)d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint64_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
        before += (uint32_t)w < wave ? wsum[w] : 0;
        total += wsum[w];
    }
    uint64_t run = before + x - mine;   // units before chunk lo
    if (quad) {
        uint64_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[k] = run * 16;
            run += s4[k];
        }
        if (per == 4 && hi == lo + 4 && !((uintptr_t)(chunk_off + lo) & 15)) {
            ulonglong2 *dst = reinterpret_cast<ulonglong2 *>(chunk_off + lo);
            dst[0] = make_ulonglong2(o[0], o[1]);
            dst[1] = make_ulonglong2(o[2], o[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (lo + k < hi) chunk_off[lo + k] = o[k];
            }
        }
    } else {
        for (uint32_t i = lo; i < hi; ++i) {
            chunk_off[i] = run * 16;
            run += sz[i];
        }
    }
    if (tid == 0) write_header(a, seg, total * 16);
    write_index_tail(a, seg, tid, kScanThreads);
}

// ----------------------------------------------------------------- 3. pack

typedef __attribute__((address_space(3))) uint32_t lds_word;

// LDS byte address of a shared-memory pointer.
template <class T>
__device__ __forceinline__ uint32_t lds_addr(T *p) {
    return (uint32_t)(size_t)(lds_word *)p;
}

// OR a left-aligned code of up to 32 bits (c, zero below its last bit) into
// a zeroed LDS bit buffer (MSB first).  The position is an absolute LDS bit
// address (the buffer's byte address times 8 plus the bit position in the
// buffer): the word address is then a shift and a mask, with no base to add.
// The code spans at most two words; OR-ing the (possibly zero) second word
// keeps the step branch-free.  The hardware shifts take the position modulo 32.
__device__ __forceinline__ void or_code32_at(uint32_t abs_bit, uint32_t c) {
    lds_word *p = (lds_word *)(size_t)((abs_bit >> 3) & ~3u);
    __hip_atomic_fetch_or(p, c >> (abs_bit & 31u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_or(p + 1, __builtin_amdgcn_alignbit(c, 0u, abs_bit), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Same for a left-aligned code of up to 64 bits held as hi:lo (three words),
// at a bit position relative to buf.
__device__ __forceinline__ void or_code64(uint32_t *buf, uint32_t pos, uint32_t hi, uint32_t lo) {
    const uint32_t w = pos >> 5;
    atomicOr(&buf[w], hi >> (pos & 31u));
    atomicOr(&buf[w + 1], __builtin_amdgcn_alignbit(hi, lo, pos));
    atomicOr(&buf[w + 2], __builtin_amdgcn_alignbit(lo, 0u, pos));
}

// Chunks per stream up to which a pack launch places the chunks itself.
constexpr uint32_t kPlaceMaxChunks = 4096;
constexpr int kPlaceLoads = kPlaceMaxChunks / kThreads;

// Placement by the pack launch, step 1: this thread's share of the sizes of
// the stream's chunks before chunk p (kPlaceLoads loads, all in flight, from
// the sizes kernel's output in L2).  Issued before the chunk's own loads.
__device__ __forceinline__ void place_issue(const EncodeArgs &a, const ChunkPos &p, uint32_t tid,
                                           uint32_t (&szv)[kPlaceLoads]) {
    const uint32_t *sz = a.sizes + (uint64_t)p.seg * a.chunks_per_seg;
    static_for<0, kPlaceLoads>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        const uint32_t i = tid + (uint32_t)k * kThreads;
        szv[k] = i < p.lc ? sz[i] : 0u;
    });
}

// Step 2 (the whole workgroup): the 16-byte units before chunk p, summed
// over the workgroup; thread 0 records chunk_off[lc], the stream's last
// chunk writes the header and its first chunk the index tail.  Returns the
// byte offset of the chunk's payload in its stream.
__device__ __forceinline__ uint64_t place_finish(const EncodeArgs &a, const ChunkPos &p, uint32_t tid, uint32_t lane,
                                                 uint32_t wave, const uint32_t (&szv)[kPlaceLoads],
                                                 uint32_t *red) {
    uint32_t x = 0;
    static_for<0, kPlaceLoads>([&](auto kc) __attribute__((always_inline)) { x += szv[decltype(kc)::value]; });
    x = wave_incl_scan(x);
    if (lane == 63) red[wave] = x;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) before += red[w];
    if (tid == 0) {
        reinterpret_cast<uint64_t *>(p.out + kHeaderBytes)[p.lc] = (uint64_t)before * 16;
        if (p.lc == a.chunks_per_seg - 1)
            write_header(a, p.seg, ((uint64_t)before + a.sizes[(uint64_t)p.seg * a.chunks_per_seg + p.lc]) * 16);
    }
    if (p.lc == 0) write_index_tail(a, p.seg, tid, kThreads);
    return (uint64_t)a.payload_offset + (uint64_t)before * 16;
}

// Byte offset of the chunk's payload in its stream, or ~0 when the chunk
// must not be written (the stream does not fit in out_cap).  `placed` is
// place_finish's result when this launch places the chunks itself;
// otherwise chunk_off[] was written by an earlier launch.
__device__ __forceinline__ uint64_t chunk_dst(const EncodeArgs &a, const ChunkPos &p, uint32_t units,
                                              uint64_t placed) {
    const uint64_t at = a.place_in_pack
                            ? placed
                            : (uint64_t)a.payload_offset + reinterpret_cast<const uint64_t *>(p.out + kHeaderBytes)[p.lc];
    const uint64_t end = at + (uint64_t)units * 16;
    return end > a.out_cap ? ~0ull : at;
}

// Staged packing, for chunks of up to 4 rows (16384 symbols) and codes of up
// to 26 bits.  Every 32-bit LUT entry (code left-aligned, length in the low
// 6 bits) is read once; each pair of codes is kept in registers as one
// left-aligned code with its length byte, four lengths to a register.  A
// piece with a pair longer than 32 bits (it needs a code of more than 16
// bits: rare for Huffman codebooks, impossible for QLC) is placed code by
// code from its bytes instead.  The whole chunk is packed
// into an LDS stage of at most kStageCap bytes; a chunk that does not fit
// (codes far longer than the codebook's typical ones) is left to the
// row-by-row packer, launched after this one when the cap can bind.

constexpr uint32_t kStageCap = 28 * 1024;   // LDS stage of the staged packer

template <int ROWS>
struct PairCache {
    uint32_t c[ROWS][kPiece / 2];     // pair codes, left-aligned (exact when the pair has <= 32 bits)
    uint32_t pk[ROWS][kPiece / 8];    // pair lengths (up to 52), one byte each
};

// Pass 1 over row r: cache the pairs; returns the piece's bit length and
// sets wide when a pair exceeds 32 bits.  All 16 bytes are looked up; bytes
// past the end of a piece are cleared afterwards by clear_tail.
template <int ROWS, bool WIDE>
__device__ __forceinline__ uint32_t cache_row(PairCache<ROWS> &cc, int r, const uint4 &v, const uint32_t *lut32,
                                              bool &wide) {
    uint32_t pk[2] = {0, 0}, mx = 0;
    static_for<0, kPiece / 2>([&](auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value;
        const uint32_t e1 = lut32[byte_k<2 * p>(v)], e2 = lut32[byte_k<2 * p + 1>(v)];
        const uint32_t l12 = (e1 & 63u) + (e2 & 63u);
        // the first code has at most 26 bits: the shift takes e1's low 5 bits
        cc.c[r][p] = (e1 & ~63u) | ((e2 & ~63u) >> (e1 & 31u));
        pk[p >> 2] |= l12 << (8 * (p & 3));
        if constexpr (!WIDE) mx = max(mx, l12);
    });
    cc.pk[r][0] = pk[0];
    cc.pk[r][1] = pk[1];
    if constexpr (WIDE) {
        // a length byte above 32, from the packed bytes (at most 52 each:
        // adding 95 sets bit 7 exactly then, with no carry into the next
        // byte).  A running maximum over the pairs kept 24 more registers
        // live through the packer (114 against 90) and cost a CU one of its
        // five workgroups.
        wide = (((pk[0] + 0x5f5f5f5fu) | (pk[1] + 0x5f5f5f5fu)) & 0x80808080u) != 0u;
    } else {
        wide = mx > 32u;   // (never: codes of at most 16 bits; unused)
    }
    return __builtin_amdgcn_sad_u8(pk[0], 0u, __builtin_amdgcn_sad_u8(pk[1], 0u, 0u));
}

// Drop the symbols at and after byte vb of a piece (vb < 16) from row r's
// cache; returns the piece's new bit length.
template <int ROWS>
__device__ __forceinline__ uint32_t clear_tail(PairCache<ROWS> &cc, int r, const uint4 &v_in, uint32_t vb,
                                               const uint32_t *lut32) {
    // Opaque copies: the compiler must not keep pass 1's table entries or
    // addresses alive for this rare path (it recomputes them here instead).
    uint4 v = v_in;
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    asm volatile("" ::: "memory");
    static_for<0, kPiece / 2>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        constexpr uint32_t sh = 8 * (u & 3);
        if ((uint32_t)(2 * u + 1) >= vb) {   // the pair keeps at most its first code
            const uint32_t e1 = (uint32_t)(2 * u) < vb ? lut32[byte_k<2 * u>(v)] : 0u;
            cc.c[r][u] = e1 & ~63u;
            cc.pk[r][u >> 2] = (cc.pk[r][u >> 2] & ~(0xffu << sh)) | ((e1 & 63u) << sh);
        }
    });
    return __builtin_amdgcn_sad_u8(cc.pk[r][0], 0u, __builtin_amdgcn_sad_u8(cc.pk[r][1], 0u, 0u));
}

// Pass 2 over row r: OR the piece's codes into LDS from absolute bit address
// pos (the stage's byte address is a multiple of 16, so word boundaries of
// the stage and of the absolute address coincide).  A wide piece is placed
// code by code from its vb bytes, read again from the input (rare, and
// cheaper than keeping every piece's bytes in registers).
template <int ROWS, bool WIDE>
__device__ __forceinline__ void emit_row(const PairCache<ROWS> &cc, int r, uint32_t pos, bool wide,
                                         const uint8_t *piece, uint32_t vb, const uint32_t *lut32) {
    if (!WIDE || !wide) {
        static_for<0, kPiece / 2>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            or_code32_at(pos, cc.c[r][u]);
            pos += (cc.pk[r][u >> 2] >> (8 * (u & 3))) & 0xffu;
        });
    } else {
        // (a piece past the segment's end reads nothing)
        const uint4 v = vb ? *reinterpret_cast<const uint4 *>(piece) : make_uint4(0u, 0u, 0u, 0u);
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            const uint32_t e = (uint32_t)k < vb ? lut32[byte_k<k>(v)] : 0u;
            or_code32_at(pos, e & ~63u);
            pos += e & 63u;
        });
    }
}

// Row-by-row packing inside the staged packer's stage, for a chunk whose
// packed bits do not fit it (codes far longer than the codebook's typical
// ones): each row of 4096 codes is ORed into the zeroed stage after the
// previous row's partial last word (the carry), then its whole words are
// stored.  A row needs at most kRowSyms * 26 / 32 words plus the carry, the
// padding to 16 bytes and the spare word (under 8), which the launch checks
// against the stage.
template <int ROWS, bool WIDE>
__device__ __forceinline__ void pack_rows_in_stage(const PairCache<ROWS> &cc, const uint32_t (&excl)[ROWS],
                                                   const uint32_t (&row_start)[ROWS], const uint32_t (&row_bits)[ROWS],
                                                   const bool (&wide)[ROWS], const uint32_t (&vb)[ROWS],
                                                   const uint8_t *src, uint32_t units, uint32_t *stage,
                                                   uint32_t *dst, uint32_t tid, const uint32_t *lut32) {
    const uint32_t base_bit = lds_addr(stage) * 8;
    const uint32_t total_words = units * 4;
    uint32_t carry = 0;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        constexpr bool last = r == ROWS - 1;
        const uint32_t rs = row_start[r], re = rs + row_bits[r];
        const uint32_t wbase = rs >> 5;
        const uint32_t nbuf = (last ? total_words : (re + 31) >> 5) - wbase;
        // the row's words plus the spare word a two-word OR may touch
        for (uint32_t i = tid; i < nbuf + 1; i += kThreads) stage[i] = i == 0 ? carry : 0u;
        __syncthreads();
        emit_row<ROWS, WIDE>(cc, r, base_bit + excl[r] - wbase * 32, wide[r], src + (uint32_t)(r * kThreads + tid) * kPiece,
                             vb[r], lut32);
        __syncthreads();
        const uint32_t nwrite = last ? nbuf : (re >> 5) - wbase;
        for (uint32_t i = tid; i < nwrite; i += kThreads) dst[wbase + i] = stage[i];
        if (!last) {
            carry = (re & 31) ? stage[(re >> 5) - wbase] : 0u;
            __syncthreads();
        }
    });
}

// A chunk fits the staged packer when its 16-byte groups plus the spare
// group the two-word ORs may touch fit the stage.
__device__ __forceinline__ bool fits_stage(const EncodeArgs &a, uint32_t units) {
    return units + 1 <= a.stage_bytes / 16;
}

// WIDE: the codebook has codes of more than 16 bits, so a pair can exceed 32.
template <int ROWS, bool WIDE>
__global__ __launch_bounds__(kThreads, 4) void encode_pack_staged_kernel(const EncodeArgs a) {
    extern __shared__ uint4 stage4[];
    __shared__ uint32_t lut32[256];
    __shared__ uint32_t wave_tot[ROWS][kThreads / 64];

    __shared__ uint32_t red[kThreads / 64];

    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const ChunkPos p = chunk_pos(a, blockIdx.x);
    // a table the host never saw may have codes too long for the 32-bit
    // entries (then all zero): its chunks go to the row-by-row packer
    const bool skip = a.tables_unread && seg_tables<EncodeArgs>(p.seg)->max_len > (uint32_t)kNarrowMaxLen;
    uint32_t szv[kPlaceLoads];
    if (a.place_in_pack) place_issue(a, p, tid, szv);
    uint4 v[ROWS];
    uint32_t vb[ROWS];
    if (!skip) load_pieces<ROWS>(p.src, p.cn, tid, v, vb);
    // uniform over the launch; every chunk is placed, also those packed later
    const uint64_t placed = a.place_in_pack ? place_finish(a, p, tid, lane, wave, szv, red) : 0;
    if (skip) return;
    lut32[tid] = seg_tables<EncodeArgs>(p.seg)->enc32[tid];
    __syncthreads();

    PairCache<ROWS> cc;
    uint32_t plen[ROWS];
    bool wide[ROWS];
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        plen[r] = cache_row<ROWS, WIDE>(cc, r, v[r], lut32, wide[r]);
    });
    if (p.cn != (uint32_t)(ROWS * kRowSyms)) {   // the segment's last chunk: drop missing symbols
        static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            if (vb[r] < (uint32_t)kPiece) plen[r] = clear_tail<ROWS>(cc, r, v[r], vb[r], lut32);
        });
    }
    uint32_t excl[ROWS], row_start[ROWS], row_bits[ROWS];
    const uint32_t chunk_bits = scan_pieces<ROWS>(plen, lane, wave, wave_tot, excl, row_start, row_bits);
    const uint32_t units = (chunk_bits + 127) >> 7;
    if (a.sized) {
        // what the sizes launch would have written; a size that differs from
        // the chunk's own (made for another codebook or input) is flagged
        write_sub_end<ROWS>(a, p, tid, excl, plen);
        if (tid == 0 && units != a.sizes[blockIdx.x])
            or_status(a.status ? a.status + p.seg : nullptr, EC_S_CODEBOOK_MISMATCH);
    }
    const uint64_t dst_at = chunk_dst(a, p, units, placed);
    // uniform over the workgroup: a chunk that does not fit is packed row by
    // row, here or (without staged_rows) by the row packer that follows
    if (dst_at == ~0ull) return;
    if (!fits_stage(a, units)) {
        if (a.staged_rows)
            pack_rows_in_stage<ROWS, WIDE>(cc, excl, row_start, row_bits, wide, vb, p.src, units,
                                           reinterpret_cast<uint32_t *>(stage4),
                                           reinterpret_cast<uint32_t *>(p.out + dst_at), tid, lut32);
        return;
    }

    for (uint32_t i = tid; i < units + 1; i += kThreads) stage4[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    const uint32_t base_bit = lds_addr(stage4) * 8;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        emit_row<ROWS, WIDE>(cc, r, base_bit + excl[r], wide[r], p.src + (uint32_t)(r * kThreads + tid) * kPiece,
                             vb[r], lut32);
    });
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(p.out + dst_at);
    for (uint32_t i = tid; i < units; i += kThreads) dst[i] = stage4[i];
}

// Row-by-row packing, any chunk size and code length up to 40 bits: each
// row of 4096 symbols is looked up (64-bit LUT entries), packed into LDS and
// stored; the partial last word is carried to the next row.
template <int ROWS>
__global__ __launch_bounds__(kThreads) void encode_pack_rows_kernel(const EncodeArgs a) {
    extern __shared__ uint32_t rowbuf[];
    __shared__ uint64_t lut64[256];
    __shared__ uint32_t wave_tot[ROWS][kThreads / 64];

    __shared__ uint32_t red[kThreads / 64];

    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const ChunkPos p = chunk_pos(a, blockIdx.x);
    // after the staged packer: only the chunks it left (the staged packer
    // then placed every chunk, so place_in_pack is 0 here)
    if (a.stage_bytes && (a.staged_rows || fits_stage(a, a.sizes[blockIdx.x])) &&
        !(a.tables_unread && seg_tables<EncodeArgs>(p.seg)->max_len > (uint32_t)kNarrowMaxLen))
        return;
    uint32_t szv[kPlaceLoads];
    if (a.place_in_pack) place_issue(a, p, tid, szv);
    uint4 v[ROWS];
    uint32_t vb[ROWS];
    load_pieces<ROWS>(p.src, p.cn, tid, v, vb);
    const uint64_t placed = a.place_in_pack ? place_finish(a, p, tid, lane, wave, szv, red) : 0;
    lut64[tid] = seg_tables<EncodeArgs>(p.seg)->enc64[tid];
    __syncthreads();

    uint32_t plen[ROWS];
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        uint32_t x = 0;
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            x += (uint32_t)k < vb[r] ? (uint32_t)lut64[byte_k<k>(v[r])] & 0xffu : 0u;
        });
        plen[r] = x;
    });
    uint32_t excl[ROWS], row_start[ROWS], row_bits[ROWS];
    const uint32_t chunk_bits = scan_pieces<ROWS>(plen, lane, wave, wave_tot, excl, row_start, row_bits);
    const uint32_t units = (chunk_bits + 127) >> 7;
    const uint64_t dst_at = chunk_dst(a, p, units, placed);
    if (dst_at == ~0ull) return;   // uniform over the workgroup: nobody reaches a later barrier

    uint32_t *dst = reinterpret_cast<uint32_t *>(p.out + dst_at);
    const uint32_t total_words = units * 4;
    uint32_t carry = 0;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        constexpr bool last = r == ROWS - 1;
        const uint32_t rs = row_start[r], re = rs + row_bits[r];
        const uint32_t wbase = rs >> 5;
        const uint32_t nbuf = (last ? total_words : (re + 31) >> 5) - wbase;
        for (uint32_t i = tid; i < nbuf; i += kThreads) rowbuf[i] = i == 0 ? carry : 0u;
        __syncthreads();
        uint32_t pos = excl[r] - wbase * 32;
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            if ((uint32_t)k < vb[r]) {
                const uint64_t e = lut64[byte_k<k>(v[r])];
                or_code64(rowbuf, pos, (uint32_t)(e >> 32), (uint32_t)e & ~0xffu);
                pos += (uint32_t)e & 0xffu;
            }
        });
        __syncthreads();
        const uint32_t nwrite = last ? nbuf : (re >> 5) - wbase;
        for (uint32_t i = tid; i < nwrite; i += kThreads) dst[wbase + i] = rowbuf[i];
        if (!last) {
            carry = (re & 31) ? rowbuf[(re >> 5) - wbase] : 0u;
            __syncthreads();
        }
    });
}

// ---------------------------------------------------------------- launches

template <int ROWS>
hipError_t launch_chunks(const EncodeArgs &a_in, uint32_t n_chunks, hipStream_t s) {
    EncodeArgs a = a_in;
    if (!a.sized) hipLaunchKernelGGL((encode_sizes_kernel<ROWS>), dim3(n_chunks), dim3(kThreads), 0, s, a);
    // short streams: the first pack launch places the chunks itself
    const bool place = a.chunks_per_seg <= kPlaceMaxChunks;
    a.place_in_pack = place ? 1u : 0u;
    if (!place) hipLaunchKernelGGL(encode_offsets_kernel, dim3(a.n_seg), dim3(kScanThreads), 0, s, a);
    // row buffer of the row-by-row packer: one row's bits plus the carried
    // word, the final padding and the spare words the three-word ORs may touch
    const uint32_t rows_lds = (kRowSyms * a.max_len / 32 + 8) * 4;
    bool all_staged = false;
    a.stage_bytes = 0;
    a.staged_rows = 0;
    // tables the host never read: staged packing for the chunks whose table
    // has 32-bit entries, sized for the longest such code
    const uint32_t narrow_len = a.tables_unread ? (uint32_t)kNarrowMaxLen : a.max_len;
    if constexpr (ROWS <= 4) {
        if (narrow_len <= (uint32_t)kNarrowMaxLen) {
            // stage: the worst-case chunk plus a spare group, capped
            const uint32_t worst = ((a.chunk_symbols * narrow_len + 127) / 128 + 1) * 16;
            a.stage_bytes = worst < kStageCap ? worst : kStageCap;
            // a chunk that overflows the stage: packed row by row in it when a
            // row of the longest narrow codes (plus carry and spare words) fits
            a.staged_rows = (kRowSyms * narrow_len / 32 + 8) * 4 <= a.stage_bytes ? 1u : 0u;
            all_staged = (worst <= kStageCap || a.staged_rows) && !a.tables_unread;
            if (narrow_len > 16)
                hipLaunchKernelGGL((encode_pack_staged_kernel<ROWS, true>), dim3(n_chunks), dim3(kThreads),
                                   a.stage_bytes, s, a);
            else
                hipLaunchKernelGGL((encode_pack_staged_kernel<ROWS, false>), dim3(n_chunks), dim3(kThreads),
                                   a.stage_bytes, s, a);
            a.place_in_pack = 0;   // the chunks are placed; the row packer reads chunk_off[]
        }
    }
    if (!all_staged)
        hipLaunchKernelGGL((encode_pack_rows_kernel<ROWS>), dim3(n_chunks), dim3(kThreads), rows_lds, s, a);
    return hipGetLastError();
}

}  // namespace

bool encode_sized_supported(uint32_t chunk_symbols, uint32_t max_len) {
    if (chunk_symbols > 4 * (uint32_t)kRowSyms || max_len > (uint32_t)kNarrowMaxLen) return false;
    // the staged packer takes every chunk (the same test as launch_chunks)
    const uint32_t worst = ((chunk_symbols * max_len + 127) / 128 + 1) * 16;
    const uint32_t stage = worst < kStageCap ? worst : kStageCap;
    return worst <= kStageCap || (kRowSyms * max_len / 32 + 8) * 4 <= stage;
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s) {
    const uint32_t n_chunks = a.n_seg * a.chunks_per_seg;
    if (n_chunks == 0) {   // header only
        hipLaunchKernelGGL(encode_offsets_kernel, dim3(a.n_seg), dim3(kScanThreads), 0, s, a);
        return hipGetLastError();
    }
    const uint32_t rows = (a.chunk_symbols + kRowSyms - 1) / kRowSyms;
    if (rows <= 1) return launch_chunks<1>(a, n_chunks, s);
    if (rows <= 2) return launch_chunks<2>(a, n_chunks, s);
    if (rows <= 4) return launch_chunks<4>(a, n_chunks, s);
    if (rows <= 8) return launch_chunks<8>(a, n_chunks, s);
    return launch_chunks<16>(a, n_chunks, s);
}

}  // namespace ec
