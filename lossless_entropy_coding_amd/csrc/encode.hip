// Chunked fixed-codebook encoder.
//
// One workgroup (256 threads, four wave64s) codes one chunk of C symbols in a
// single pass over HBM:
//   1. take a ticket (chunks are handed out in launch order, so every chunk
//      a workgroup waits for below is already running);
//   2. load the chunk as 16-byte pieces, piece q = r * 256 + thread, so each
//      load instruction of a wave reads 1 KiB of contiguous bytes;
//   3. sum each piece's code lengths from the codebook's LUT held in LDS;
//   4. exclusive scan of piece lengths (wave scan + LDS across the four
//      waves) gives every piece's bit offset in the chunk and the end bit of
//      each 256-symbol sub-chunk, which goes straight into the stream index;
//   5. decoupled look-back over earlier chunks' published sizes (agent-scope
//      relaxed atomics, tagged with a per-launch epoch so the flag words
//      never need clearing) gives the chunk's byte offset in the payload;
//   6. for each row of 4096 symbols the pieces OR their codes into an LDS
//      word buffer (64-bit accumulator per thread, MSB first), and the
//      workgroup stores the finished words with coalesced 32-bit stores;
//      the partial last word is carried to the next row.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kPiece = 16;                     // symbols per piece (one 16-byte load)
constexpr int kRowSyms = kThreads * kPiece;    // 4096
constexpr uint64_t kFlagAgg = 1ull << 62;      // chunk size published, prefix not yet known
constexpr uint64_t kFlagPrefix = 2ull << 62;   // inclusive prefix published
constexpr uint32_t kMaxSpins = 1u << 22;       // look-back wait bound (about 0.1-1 s)
constexpr int kLookGroups = 4;                 // look-back reads 4 x 64 predecessors per pass

// Byte K (compile-time) of a 16-byte piece, in memory order.
template <int K>
__device__ __forceinline__ uint32_t byte_k(const uint4 &v) {
    constexpr int w = K >> 2, sh = 8 * (K & 3);
    const uint32_t x = w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
    return (x >> sh) & 0xffu;
}

// Code length of byte b.
template <bool WIDE>
__device__ __forceinline__ uint32_t code_len(const uint32_t *lut32, const uint64_t *lut64, uint32_t b) {
    if (WIDE) return (uint32_t)(lut64[b] >> 56);
    return lut32[b] >> 24;
}

// Sum of the code lengths of the first vb bytes of a piece.
template <bool WIDE>
__device__ __forceinline__ uint32_t piece_len(const uint4 &v, uint32_t vb, const uint32_t *lut32,
                                              const uint64_t *lut64) {
    uint32_t x = 0;
    if (vb == kPiece) {
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) { x += code_len<WIDE>(lut32, lut64, byte_k<decltype(kc)::value>(v)); });
    } else {
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            if ((uint32_t)k < vb) x += code_len<WIDE>(lut32, lut64, byte_k<k>(v));
        });
    }
    return x;
}

// OR the l low bits of c (l <= 32) into the zeroed LDS word buffer at bit
// position pos (MSB first); a code spans at most two words, and OR-ing the
// (possibly zero) second word keeps the step branch-free.
__device__ __forceinline__ void or_bits(uint32_t *buf, uint32_t pos, uint32_t c, uint32_t l) {
    const uint32_t w = pos >> 5;
    const uint64_t v = (uint64_t)c << (64u - (pos & 31u) - l);
    atomicOr(&buf[w], (uint32_t)(v >> 32));
    atomicOr(&buf[w + 1], (uint32_t)v);
}

// OR the codes of the first vb bytes of a piece into buf from bit `bitoff`.
// All LUT entries are read first: the buffer ORs that follow are LDS stores
// the compiler cannot move table reads past.  Codes of up to 16 bits are
// joined in pairs (at most 32 bits) before they are placed.
template <bool WIDE, bool PAIRS>
__device__ __forceinline__ void emit_piece(const uint4 &v, uint32_t vb, uint32_t bitoff, const uint32_t *lut32,
                                           const uint64_t *lut64, uint32_t *buf) {
    uint32_t pos = bitoff;
    if (!WIDE) {
        uint32_t e[kPiece];
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            e[k] = (uint32_t)k < vb ? lut32[byte_k<k>(v)] : 0u;   // length 0: nothing to place
        });
        if (PAIRS) {
            static_for<0, kPiece / 2>([&](auto pc) __attribute__((always_inline)) {
                constexpr int p = decltype(pc)::value;
                const uint32_t l1 = e[2 * p] >> 24, l2 = e[2 * p + 1] >> 24;
                const uint32_t c = ((e[2 * p] & 0xffffffu) << l2) | (e[2 * p + 1] & 0xffffffu);
                const uint32_t l = l1 + l2;
                if (l) or_bits(buf, pos, c, l);
                pos += l;
            });
        } else {
            static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                const uint32_t l = e[k] >> 24;
                if (l) or_bits(buf, pos, e[k] & 0xffffffu, l);
                pos += l;
            });
        }
    } else {
        static_for<0, kPiece>([&](auto kc) __attribute__((always_inline)) {
            constexpr int k = decltype(kc)::value;
            if ((uint32_t)k < vb) {
                const uint64_t e = lut64[byte_k<k>(v)];
                const uint32_t l = (uint32_t)(e >> 56);
                const uint64_t c = e & ((1ull << 56) - 1);
                if (l > 32) {
                    or_bits(buf, pos, (uint32_t)(c >> 32), l - 32);
                    or_bits(buf, pos + (l - 32), (uint32_t)c, 32);
                } else {
                    or_bits(buf, pos, (uint32_t)c, l);
                }
                pos += l;
            }
        });
    }
}

// Header fields, chunk_off[0] and the zero fill up to the payload (and the
// embedded code lengths): written once per stream by the thread block that
// owns the stream's first chunk (or by the header-only kernel when n = 0).
__device__ __forceinline__ void write_stream_head(const EncodeArgs &a, uint32_t seg, const DevTables *tab, uint32_t tid,
                                  uint32_t nthreads) {
    uint8_t *out = a.out + (uint64_t)seg * a.out_stride;
    const uint32_t spc = a.chunk_symbols / kSub;
    const uint32_t index_end = a.sub_at + 4u * a.chunks_per_seg * spc;
    if (tid == 0) {
        uint64_t *h = reinterpret_cast<uint64_t *>(out);
        h[0] = (uint64_t)kMagic | ((uint64_t)kVersion << 32) | ((uint64_t)tab->codec << 48) |
               ((uint64_t)(a.embed_lengths ? 1 : 0) << 56);
        h[1] = a.seg_n;
        h[2] = (uint64_t)a.chunk_symbols | ((uint64_t)a.chunks_per_seg << 32);
        h[3] = a.payload_offset;
        h[5] = tab->codebook_id;
        h[6] = 0;
        h[7] = 0;
        if (a.chunks_per_seg == 0) {
            h[4] = 0;          // payload_bytes
            h[8] = 0;          // chunk_off[0]
            a.out_len[seg] = a.payload_offset;
        }
    }
    uint32_t pad_from = index_end;
    if (a.embed_lengths) {
        for (uint32_t i = tid; i < 256; i += nthreads) out[index_end + i] = tab->code_len[i];
        pad_from += 256;
    }
    for (uint32_t i = pad_from + tid; i < a.payload_offset; i += nthreads) out[i] = 0;
}

template <int ROWS, bool WIDE, bool PAIRS>
__global__ __launch_bounds__(kThreads) void encode_kernel(const EncodeArgs a) {
    extern __shared__ uint32_t rowbuf[];
    __shared__ uint64_t lut64[WIDE ? 256 : 1];
    __shared__ uint32_t lut32[WIDE ? 1 : 256];
    __shared__ uint32_t wave_tot[ROWS][kThreads / 64];
    __shared__ uint32_t s_chunk, s_excl, s_skip;

    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        const uint32_t t = add_agent(a.ticket, 1u);
        if (t == gridDim.x - 1) st_agent32(a.ticket, 0u);   // every ticket is taken: reset for the next launch
        s_chunk = t;
    }
    __syncthreads();
    const uint32_t chunk = s_chunk;
    const uint32_t seg = chunk / a.chunks_per_seg;
    const uint32_t lc = chunk - seg * a.chunks_per_seg;
    const DevTables *tab = seg_tables<EncodeArgs>(seg);
    if (WIDE)
        lut64[tid] = tab->enc64[tid];
    else
        lut32[tid] = tab->enc32[tid];

    const uint64_t first = (uint64_t)lc * a.chunk_symbols;
    const uint64_t left = a.seg_n - first;
    const uint32_t cn = left < a.chunk_symbols ? (uint32_t)left : a.chunk_symbols;
    const uint8_t *src = a.in + (uint64_t)seg * a.in_stride + first;
    uint8_t *out = a.out + (uint64_t)seg * a.out_stride;

    // 2. load pieces
    uint4 v[ROWS];
    uint32_t vb[ROWS];
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        const uint32_t off = (uint32_t)(r * kThreads + tid) * kPiece;
        vb[r] = off < cn ? min(cn - off, (uint32_t)kPiece) : 0u;
        if (vb[r] == kPiece) {
            v[r] = *reinterpret_cast<const uint4 *>(src + off);
        } else {
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < kPiece; ++k)
                if ((uint32_t)k < vb[r]) w[k >> 2] |= (uint32_t)src[off + k] << (8 * (k & 3));
            v[r] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    });
    __syncthreads();   // LUT in LDS

    // 3. piece lengths, 4. wave-inclusive scan per row
    uint32_t plen[ROWS], incl[ROWS];
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        uint32_t x = piece_len<WIDE>(v[r], vb[r], lut32, lut64);
        plen[r] = x;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t y = __shfl_up(x, d, 64);
            if (lane >= (uint32_t)d) x += y;
        }
        incl[r] = x;
        if (lane == 63) wave_tot[r][wave] = x;
    });
    __syncthreads();
    // combine the four waves: piece offsets, row starts, chunk total
    uint32_t excl[ROWS], row_start[ROWS], row_bits[ROWS];
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
    const uint32_t chunk_bits = total;

    // 5. look-back for the chunk's byte offset (in 16-byte units): wave 0
    //    reads the flags of 64 predecessors at a time, the nearest published
    //    prefix ends the walk, the sizes in between are summed
    if (wave == 0) {
        const uint32_t units = (chunk_bits + 127) >> 7;
        const uint64_t ep = (uint64_t)a.epoch << 32;
        uint32_t acc = 0;
        bool timed_out = false;
        if (lc == 0) {
            if (lane == 0) st_agent(&a.flags[chunk], kFlagPrefix | ep | units);
        } else {
            if (lane == 0) st_agent(&a.flags[chunk], kFlagAgg | ep | units);
            const int64_t first = (int64_t)(chunk - lc);    // the segment's first chunk
            int64_t top = (int64_t)chunk - 1;
            uint32_t spins = 0;
            for (;;) {
                // predecessors top - (lane + 64 g), g = 0..kLookGroups-1, all requested at once
                uint64_t f[kLookGroups];
#pragma unroll
                for (int g = 0; g < kLookGroups; ++g) {
                    const int64_t k = top - (int64_t)lane - 64 * g;
                    f[g] = k >= first ? ld_agent(&a.flags[k]) : (kFlagPrefix | ep);
                }
                bool retry = false, found = false;
                uint32_t sum = 0, whole = 0;   // sum over complete groups / their count
#pragma unroll
                for (int g = 0; g < kLookGroups; ++g) {
                    if (found || retry) break;
                    const bool valid = ((f[g] >> 32) & 0x3fffffffu) == a.epoch;
                    const uint64_t pref = __ballot(valid && (f[g] >> 62) == 2);
                    const uint64_t inval = __ballot(!valid);
                    const uint32_t stop = pref ? (uint32_t)__builtin_ctzll(pref) : 64u;
                    const uint64_t need = stop >= 63 ? ~0ull : ((2ull << stop) - 1);
                    if (inval & need) {
                        retry = true;
                        break;
                    }
                    uint32_t v = lane <= stop ? (uint32_t)f[g] : 0u;
#pragma unroll
                    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
                    sum += v;
                    found = stop < 64;
                    whole += found ? 0u : 1u;
                }
                // groups without a published prefix are consumed; the walk
                // continues below them (or waits on the group that is not ready)
                acc += sum;
                top -= 64 * (int64_t)whole;
                if (found) break;
                if (retry) {
                    // bounded wait: a chunk that never publishes is a bug, not a hang
                    if (++spins > kMaxSpins) {
                        timed_out = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (lane == 0 && !timed_out) st_agent(&a.flags[chunk], kFlagPrefix | ep | (uint64_t)(acc + units));
        }
        if (lane == 0) {
            s_excl = acc;
            uint64_t *chunk_off = reinterpret_cast<uint64_t *>(out + kHeaderBytes);
            chunk_off[lc] = (uint64_t)acc * 16;
            const uint64_t end = (uint64_t)a.payload_offset + ((uint64_t)acc + units) * 16;
            s_skip = end > a.out_cap || timed_out;
            if (end > a.out_cap) or_status(a.status ? a.status + seg : nullptr, EC_S_CAPACITY);
            if (timed_out) or_status(a.status ? a.status + seg : nullptr, EC_S_INTERNAL);
            if (lc == a.chunks_per_seg - 1) {
                chunk_off[lc + 1] = ((uint64_t)acc + units) * 16;
                reinterpret_cast<uint64_t *>(out)[4] = ((uint64_t)acc + units) * 16;   // payload_bytes
                a.out_len[seg] = end;
            }
        }
    }
    if (lc == 0) write_stream_head(a, seg, tab, tid, kThreads);
    // sub-chunk ends: the last piece of each 256-symbol sub-chunk (written
    // after the look-back, whose flag loads would otherwise wait on them)
    const uint32_t spc = a.chunk_symbols / kSub;
    uint32_t *sub_end = reinterpret_cast<uint32_t *>(out + a.sub_at) + (uint64_t)lc * spc;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        const uint32_t q = (uint32_t)r * kThreads + tid;
        if ((tid & 15) == 15 && q < a.chunk_symbols / kPiece) sub_end[q >> 4] = excl[r] + plen[r];
    });
    __syncthreads();
    if (s_skip) return;

    // 6. pack rows into LDS and store finished words
    uint32_t *dst = reinterpret_cast<uint32_t *>(out + a.payload_offset + (uint64_t)s_excl * 16);
    const uint32_t total_words = ((chunk_bits + 127) >> 7) * 4;
    uint32_t carry = 0;
    static_for<0, ROWS>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        constexpr bool last = r == ROWS - 1;
        const uint32_t rs = row_start[r], re = rs + row_bits[r];
        const uint32_t wbase = rs >> 5;
        const uint32_t nbuf = (last ? total_words : (re + 31) >> 5) - wbase;
        for (uint32_t i = tid; i < nbuf; i += kThreads) rowbuf[i] = i == 0 ? carry : 0u;
        __syncthreads();
        if (plen[r]) emit_piece<WIDE, PAIRS>(v[r], vb[r], excl[r] - wbase * 32, lut32, lut64, rowbuf);
        __syncthreads();
        const uint32_t nwrite = last ? nbuf : (re >> 5) - wbase;
        for (uint32_t i = tid; i < nwrite; i += kThreads) dst[wbase + i] = rowbuf[i];
        if (!last) {
            carry = (re & 31) ? rowbuf[(re >> 5) - wbase] : 0u;
            __syncthreads();
        }
    });
}

__global__ void header_only_kernel(const EncodeArgs a) {
    const uint32_t seg = blockIdx.x;
    write_stream_head(a, seg, seg_tables<EncodeArgs>(seg), threadIdx.x, blockDim.x);
}

template <int ROWS>
hipError_t launch_rows(const EncodeArgs &a, uint32_t max_len, uint32_t grid, uint32_t lds, hipStream_t s) {
    if (max_len > (uint32_t)kNarrowMaxLen)
        hipLaunchKernelGGL((encode_kernel<ROWS, true, false>), dim3(grid), dim3(kThreads), lds, s, a);
    else if (max_len > 16)
        hipLaunchKernelGGL((encode_kernel<ROWS, false, false>), dim3(grid), dim3(kThreads), lds, s, a);
    else
        hipLaunchKernelGGL((encode_kernel<ROWS, false, true>), dim3(grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, uint32_t /*codec*/, hipStream_t s) {
    const uint32_t grid = a.n_seg * a.chunks_per_seg;
    const uint32_t rows = (a.chunk_symbols + kRowSyms - 1) / kRowSyms;
    // row buffer: one row's bits plus the carried word, the final padding and
    // the spare word the two-word ORs may touch
    const uint32_t lds = (kRowSyms * a.max_len / 32 + 8) * 4;
    if (rows <= 1) return launch_rows<1>(a, a.max_len, grid, lds, s);
    if (rows <= 2) return launch_rows<2>(a, a.max_len, grid, lds, s);
    if (rows <= 4) return launch_rows<4>(a, a.max_len, grid, lds, s);
    if (rows <= 8) return launch_rows<8>(a, a.max_len, grid, lds, s);
    return launch_rows<16>(a, a.max_len, grid, lds, s);
}

hipError_t launch_header_only(const EncodeArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(header_only_kernel, dim3(a.n_seg), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ec
