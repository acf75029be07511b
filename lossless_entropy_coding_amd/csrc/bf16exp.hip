// Exponent coding of BF16 tensors ("ZipCCL: Efficient Lossless Data
// Compression of Communication Collectives for Accelerating LLM Training",
// methodology B and C): every value splits into a sign-and-mantissa byte and
// its 8-bit exponent; the seven exponents of the table get the 3-bit codes
// 1..7, any other exponent code 0 and a place, in value order, in the escape
// array.  The codes are kept as three 1-bit planes (bit k of value i's code
// is bit i & 7 of byte i >> 3 of plane k), so every section is written and
// read with coalesced stores and loads.
//
// Encode, two launches:
//   1. bf16_encode_kernel (one workgroup per chunk): each thread takes
//      pieces of 16 values (two 16-byte loads), writes their sign-mantissa
//      bytes (one 16-byte store) and two bytes of each plane, and stages the chunk's escaped
//      exponents, in value order, in scratch (each row's gathered in LDS
//      first, then stored contiguously); records the chunk's count.
//   2. bf16_place_kernel (one workgroup per chunk): sums the counts of the
//      earlier chunks, records esc_off[c], copies the chunk's escapes to
//      their place; the last chunk writes the header, the first the zero
//      fill between sections.
// Decode (persistent workgroups, whole chunks each, row by row): a chunk's
// escapes start at esc_off[c]; each row's code-0 values advance the
// position, which must reach esc_off[c + 1] exactly.  A row's escapes are
// loaded into LDS with contiguous loads, then taken in value order.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kBfThreads = 256;
constexpr uint32_t kBfPiece = 16;                         // values per thread and row (two 16-byte loads)
constexpr uint32_t kBfRowVals = kBfThreads * kBfPiece;    // 4096
constexpr uint32_t kBfChunkUnit = 2048;                   // a chunk holds a multiple of this many values
constexpr uint32_t kBfMagic = 0x36314245u;                // "EB16"
constexpr uint32_t kBfVersion = 1;

// Exclusive position of this thread's count in the workgroup (thread order)
// and the workgroup's total; wsum holds one word per wave.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t lane, uint32_t wave, uint32_t *wsum,
                                                    uint32_t *total) {
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kBfThreads / 64; ++w) {
        before += (uint32_t)w < wave ? wsum[w] : 0u;
        t += wsum[w];
    }
    __syncthreads();   // wsum is reused by the next scan
    *total = t;
    return before + incl - x;
}

// The 16 values of a piece (count nv <= 16; the others read as 0).
__device__ __forceinline__ void load_piece(const uint16_t *src, uint32_t nv, uint32_t (&v)[kBfPiece]) {
    if (nv == kBfPiece) {
        const uint4 q0 = reinterpret_cast<const uint4 *>(src)[0], q1 = reinterpret_cast<const uint4 *>(src)[1];
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v[2 * k] = w[k] & 0xffffu;
            v[2 * k + 1] = w[k] >> 16;
        }
    } else {
#pragma unroll
        for (uint32_t j = 0; j < kBfPiece; ++j) v[j] = j < nv ? (uint32_t)src[j] : 0u;
    }
}

__global__ __launch_bounds__(kBfThreads, 8) void bf16_encode_kernel(const BfArgs a) {
    __shared__ uint8_t code_of[256];
    __shared__ uint8_t esc_row[kBfRowVals];   // one row's escapes (reused after the next row's scan barriers)
    __shared__ uint32_t wsum[kBfThreads / 64];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t cd = 0;
#pragma unroll
    for (int k = 1; k <= 7; ++k) cd = a.table[k] == tid ? (uint32_t)k : cd;
    code_of[tid] = (uint8_t)cd;
    __syncthreads();

    const uint32_t c = blockIdx.x;
    const uint64_t c0 = (uint64_t)c * a.chunk;
    const uint32_t cn = (uint32_t)min((uint64_t)a.chunk, a.n - c0);
    const uint32_t rows = (cn + kBfRowVals - 1) / kBfRowVals;
    uint8_t *sm_out = a.out + a.sm_at + c0;
    uint8_t *plane = a.out + a.plane_at + (c0 >> 3);
    uint8_t *esc_tmp = a.esc_tmp + c0;
    uint32_t chunk_esc = 0;   // escapes of the chunk's earlier rows (uniform)
    for (uint32_t r = 0; r < rows; ++r) {
        const uint32_t i = (r * kBfThreads + tid) * kBfPiece;   // first value of the piece in the chunk
        const uint32_t nv = i < cn ? min(cn - i, kBfPiece) : 0u;
        uint32_t v[kBfPiece];
        load_piece(a.in + c0 + i, nv, v);
        uint32_t e[kBfPiece];
        uint32_t smw[kBfPiece / 4] = {0, 0, 0, 0}, p0 = 0, p1 = 0, p2 = 0, escm = 0;
#pragma unroll
        for (uint32_t j = 0; j < kBfPiece; ++j) {
            e[j] = (v[j] >> 7) & 0xffu;
            const uint32_t s = ((v[j] >> 8) & 0x80u) | (v[j] & 0x7fu);
            smw[j / 4] |= s << (8 * (j % 4));
            const uint32_t k = j < nv ? (uint32_t)code_of[e[j]] : 0u;
            p0 |= (k & 1u) << j;
            p1 |= ((k >> 1) & 1u) << j;
            p2 |= (k >> 2) << j;
            escm |= (j < nv && k == 0u) ? 1u << j : 0u;
        }
        if (nv == kBfPiece) {
            *reinterpret_cast<uint4 *>(sm_out + i) = make_uint4(smw[0], smw[1], smw[2], smw[3]);
        } else {
            for (uint32_t j = 0; j < nv; ++j) sm_out[i + j] = (uint8_t)(smw[j / 4] >> (8 * (j % 4)));
        }
        // plane bytes: two for a piece with values past its first eight (a
        // 2-byte aligned pair: i is a multiple of 16), else one
        if (nv > 8) {
            *reinterpret_cast<uint16_t *>(plane + (i >> 3)) = (uint16_t)p0;
            *reinterpret_cast<uint16_t *>(plane + a.plane_bytes + (i >> 3)) = (uint16_t)p1;
            *reinterpret_cast<uint16_t *>(plane + 2 * a.plane_bytes + (i >> 3)) = (uint16_t)p2;
        } else if (nv) {
            plane[i >> 3] = (uint8_t)p0;
            plane[a.plane_bytes + (i >> 3)] = (uint8_t)p1;
            plane[2 * a.plane_bytes + (i >> 3)] = (uint8_t)p2;
        }
        // the row's escapes, in value order: each thread's into LDS at its
        // scanned place, then the row's bytes to scratch with contiguous
        // stores (a byte store per escaped value would issue up to sixteen
        // divergent stores per row)
        uint32_t row_total;
        uint32_t pos = block_excl_scan(__popc(escm), lane, wave, wsum, &row_total);
#pragma unroll
        for (uint32_t j = 0; j < kBfPiece; ++j) {
            if (escm & (1u << j)) esc_row[pos++] = (uint8_t)e[j];
        }
        __syncthreads();
        for (uint32_t k = tid; k < row_total; k += kBfThreads) esc_tmp[chunk_esc + k] = esc_row[k];
        chunk_esc += row_total;
    }
    if (tid == 0) a.counts[c] = chunk_esc;
}

__global__ __launch_bounds__(kBfThreads) void bf16_place_kernel(const BfArgs a) {
    __shared__ uint32_t wsum[kBfThreads / 64];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t c = blockIdx.x;   // with no chunk at all, one workgroup writes the header
    uint32_t x = 0;
    for (uint32_t k = tid; k < c; k += kBfThreads) x += a.counts[k];
    uint32_t before;
    (void)block_excl_scan(x, lane, wave, wsum, &before);
    const uint32_t mine = c < a.n_chunks ? a.counts[c] : 0u;
    uint64_t *esc_off = reinterpret_cast<uint64_t *>(a.out + kHeaderBytes);
    const uint64_t dst = a.esc_at + before;
    if (c < a.n_chunks) {
        if (tid == 0) esc_off[c] = before;
        if (dst + mine <= a.out_cap) {
            const uint8_t *src = a.esc_tmp + (uint64_t)c * a.chunk;
            for (uint32_t k = tid; k < mine; k += kBfThreads) a.out[dst + k] = src[k];
        }
    }
    if (c + 1 >= a.n_chunks && tid == 0) {   // the last chunk (or the only workgroup)
        const uint64_t total = (uint64_t)before + mine;
        esc_off[a.n_chunks] = total;
        uint64_t *h = reinterpret_cast<uint64_t *>(a.out);
        h[0] = (uint64_t)kBfMagic | ((uint64_t)kBfVersion << 32);
        h[1] = a.n;
        h[2] = (uint64_t)a.chunk | ((uint64_t)a.n_chunks << 32);
        uint64_t t = 0;
        for (int k = 6; k >= 0; --k) t = (t << 8) | a.table[1 + k];
        h[3] = t;
        h[4] = total;
        h[5] = a.sm_at;
        h[6] = a.plane_at;
        h[7] = a.esc_at;
        const uint64_t end = a.esc_at + total;
        a.out_len[0] = end;
        if (end > a.out_cap) or_status(a.status, EC_S_CAPACITY);
    }
    if (c == 0) {   // zero fill: after the index, after the sign-mantissa bytes, after each plane's bits
        const uint64_t idx_end = kHeaderBytes + 8ull * (a.n_chunks + 1);
        for (uint64_t k = idx_end + tid; k < a.sm_at; k += kBfThreads) a.out[k] = 0;
        for (uint64_t k = a.sm_at + a.n + tid; k < a.plane_at; k += kBfThreads) a.out[k] = 0;
        const uint64_t used = (a.n + 7) / 8;
        for (int p = 0; p < 3; ++p)
            for (uint64_t k = used + tid; k < a.plane_bytes; k += kBfThreads) a.out[a.plane_at + p * a.plane_bytes + k] = 0;
    }
}

// Code-0 (escaped) values among the 8 whose plane bytes are b0, b1, b2, of
// which the first nv exist.
__device__ __forceinline__ uint32_t esc_mask(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t nv) {
    return ~(b0 | b1 | b2) & ((1u << nv) - 1u);
}

__global__ __launch_bounds__(kBfThreads, 8) void bf16_decode_kernel(const BfDecArgs a) {
    __shared__ uint32_t wsum[kBfThreads / 64];
    __shared__ uint8_t esc_row[kBfRowVals];   // one row's escapes (reused after the next row's scan barriers)
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the header, read and checked by every thread (uniform)
    const uint64_t *h = reinterpret_cast<const uint64_t *>(a.in);
    const uint64_t h0 = h[0], n = h[1], h2 = h[2], tab = h[3], n_esc = h[4], sm_at = h[5], plane_at = h[6],
                   esc_at = h[7];
    const uint32_t chunk = (uint32_t)h2, n_chunks = (uint32_t)(h2 >> 32);
    bool ok = (uint32_t)h0 == kBfMagic && (h0 >> 32) == kBfVersion && n == a.n && chunk > 0 &&
              chunk % kBfChunkUnit == 0 && (uint64_t)n_chunks == (n + chunk - 1) / chunk && n_esc <= n;
    if (ok) {   // the sections where the layout puts them
        const uint64_t idx_end = kHeaderBytes + 8ull * (n_chunks + 1);
        const uint64_t e_sm = (idx_end + 255) / 256 * 256, e_pl = (e_sm + n + 15) / 16 * 16;
        const uint64_t pb = ((n + 7) / 8 + 15) / 16 * 16;
        ok = sm_at == e_sm && plane_at == e_pl && esc_at == e_pl + 3 * pb && esc_at + n_esc <= a.in_len;
    }
    if (!ok) {
        if (blockIdx.x == 0 && tid == 0) or_status(a.status, EC_S_BAD_HEADER);
        return;   // uniform over the launch
    }
    const uint64_t pb = ((n + 7) / 8 + 15) / 16 * 16;
    uint32_t table[8];
    table[0] = 0;
#pragma unroll
    for (int k = 0; k < 7; ++k) table[1 + k] = (uint32_t)(tab >> (8 * k)) & 0xffu;
    const uint8_t *plane = a.in + plane_at;
    const uint64_t *esc_off = reinterpret_cast<const uint64_t *>(a.in + kHeaderBytes);

    // persistent workgroups: whole chunks, row by row, carrying the escape position
    for (uint32_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
        const uint64_t c0 = (uint64_t)c * chunk;
        const uint32_t cn = (uint32_t)min((uint64_t)chunk, n - c0);
        const uint32_t rows = (cn + kBfRowVals - 1) / kBfRowVals;
        const uint64_t lo = esc_off[c], hi = esc_off[c + 1];
        bool bad = lo > hi || hi > n_esc;   // uniform
        uint64_t run = lo;
        for (uint32_t r = 0; r < rows; ++r) {
            const uint32_t ic = (r * kBfThreads + tid) * kBfPiece;   // first value of the piece in the chunk
            const uint64_t i = c0 + ic;
            const uint32_t nv = ic < cn ? min(cn - ic, kBfPiece) : 0u;
            // plane bits: two bytes (2-byte aligned: i is a multiple of 16)
            // for a piece with values past its first eight, else one
            uint32_t b0 = 0, b1 = 0, b2 = 0, smw[kBfPiece / 4] = {0, 0, 0, 0};
            if (nv > 8) {
                b0 = *reinterpret_cast<const uint16_t *>(plane + (i >> 3));
                b1 = *reinterpret_cast<const uint16_t *>(plane + pb + (i >> 3));
                b2 = *reinterpret_cast<const uint16_t *>(plane + 2 * pb + (i >> 3));
            } else if (nv) {
                b0 = plane[i >> 3];
                b1 = plane[pb + (i >> 3)];
                b2 = plane[2 * pb + (i >> 3)];
            }
            if (nv == kBfPiece) {
                const uint4 sv = *reinterpret_cast<const uint4 *>(a.in + sm_at + i);
                smw[0] = sv.x;
                smw[1] = sv.y;
                smw[2] = sv.z;
                smw[3] = sv.w;
            } else {
                for (uint32_t j = 0; j < nv; ++j) smw[j / 4] |= (uint32_t)a.in[sm_at + i + j] << (8 * (j % 4));
            }
            const uint32_t em = esc_mask(b0, b1, b2, nv);
            uint32_t row_esc;
            uint32_t pos = block_excl_scan(__popc(em), lane, wave, wsum, &row_esc);
            // a consistent index keeps the chunk's escapes inside its range
            bad = bad || run + row_esc > hi;
            // the row's escapes (at most one per value) into LDS with
            // contiguous loads, instead of a byte load per escaped value
            for (uint32_t k = tid; k < row_esc; k += kBfThreads)
                esc_row[k] = (!bad && run + k < n_esc) ? a.in[esc_at + run + k] : (uint8_t)0;
            __syncthreads();
            uint32_t out[kBfPiece];
#pragma unroll
            for (uint32_t j = 0; j < kBfPiece; ++j) {
                const uint32_t k = ((b0 >> j) & 1u) | (((b1 >> j) & 1u) << 1) | (((b2 >> j) & 1u) << 2);
                uint32_t e = table[k];
                if ((em >> j) & 1u) e = esc_row[pos++];
                const uint32_t sb = (smw[j / 4] >> (8 * (j % 4))) & 0xffu;
                out[j] = ((sb & 0x80u) << 8) | (e << 7) | (sb & 0x7fu);
            }
            if (nv == kBfPiece) {
                uint4 *o = reinterpret_cast<uint4 *>(a.out + i);
                o[0] = make_uint4(out[0] | (out[1] << 16), out[2] | (out[3] << 16), out[4] | (out[5] << 16),
                                  out[6] | (out[7] << 16));
                o[1] = make_uint4(out[8] | (out[9] << 16), out[10] | (out[11] << 16), out[12] | (out[13] << 16),
                                  out[14] | (out[15] << 16));
            } else {
                for (uint32_t j = 0; j < nv; ++j) a.out[i + j] = (uint16_t)out[j];
            }
            run += row_esc;
        }
        // the chunk's escapes must end exactly where the next chunk's start
        if ((bad || run != hi) && tid == 0) or_status(a.status, EC_S_CORRUPT);
    }
}

}  // namespace

hipError_t launch_bf16_encode(const BfArgs &a, hipStream_t s) {
    if (a.n_chunks) hipLaunchKernelGGL(bf16_encode_kernel, dim3(a.n_chunks), dim3(kBfThreads), 0, s, a);
    hipLaunchKernelGGL(bf16_place_kernel, dim3(a.n_chunks ? a.n_chunks : 1), dim3(kBfThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bf16_decode(const BfDecArgs &a, hipStream_t s) {
    // the chunk size is in the stream: at most one workgroup per 2048-value
    // row (no more than there can be chunks), and persistent beyond 2048
    const uint64_t rows = (a.n + kBfRowVals - 1) / kBfRowVals;
    const uint32_t grid = rows == 0 ? 1u : (uint32_t)min(rows, (uint64_t)2048);
    hipLaunchKernelGGL(bf16_decode_kernel, dim3(grid), dim3(kBfThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ec
