// Byte histogram and the PMF statistics kernels.
//
// Histogram, two launches:
//   1. histogram_kernel: each workgroup of 1024 threads takes whole 128 KiB
//      pieces of a segment (8 vectors of 16 bytes per thread, all loads in
//      flight before the first count) and counts them into one table of
//      32 columns x 256 bins in LDS: lane l adds into column l & 31, so the
//      32 lanes of one LDS pass always hit 32 different banks and two lanes
//      of one instruction meet on a counter only when they are l and l + 32
//      with equal bytes.  The table is then summed over its columns and the
//      workgroup stores its 256 partial counts (bin-major rows).
//   2. histogram_reduce_kernel: sums the partial rows of each segment into
//      the 64-bit counts, one wave per bin.
// No global atomics: same-address atomics from many workgroups serialise at
// the memory side.
//
// With chunk sizes (the single-stage design fixes the codebooks before the
// data is seen, so the pass that counts the bytes can also size the chunks
// an encode will make): a second LDS table in the counters' layout holds,
// for byte b, the code lengths of the codebooks (up to two: at bits 0 and
// 16, so that sums need no unpacking; up to four: one byte each), read at
// the counter's own address plus a constant.  Each 16-byte vector's lengths
// add up in 16-bit halves of one or two registers, the wave adds
// its lanes' sums when its 64 vectors lie in one chunk (else every lane adds
// its own), and per-chunk totals gather in LDS; after each piece they are
// stored as 16-byte units.  A chunk is a power of two of vectors that
// divides a piece, so no chunk spans two workgroups.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kHistThreads = 1024;
constexpr int kHistCols = 32;                          // counter columns (lane & 31)
constexpr int kHistWords = 256 * kHistCols;            // 32 KiB of counters per workgroup
constexpr int kHistVec = 8;                            // 16-byte loads per thread per piece
constexpr uint64_t kHistPiece = (uint64_t)kHistVec * kHistThreads;   // vectors per piece (128 KiB)

// With chunk sizes the large pieces are half as long (64 KiB): the per-byte
// length reads need registers that eight vectors in flight would take.
constexpr int kHistVecSized = 4;
constexpr uint64_t kSizedPiece = (uint64_t)kHistVecSized * kHistThreads;
constexpr uint32_t kMaxPieceChunks = kSizedPiece / 16;   // chunks of 256 symbols in a piece

// The counters, then the length table in the same layout (word 32 b + c):
// a counter and its length word are one address apart by a constant, so a
// byte's address serves both (the LDS instructions' offset field).
struct SizeSmem {
    uint4 cnt[kHistWords / 4];
    uint32_t len[kHistWords];
    uint32_t acc[kMaxSizeCodebooks][kMaxPieceChunks];   // bits per chunk of the piece
};

// Small segments take pieces of one vector per thread (16 KiB), so that
// they still spread over many compute units.
// (two workgroups per CU: at most 64 VGPRs)
// NCB: 0 (counts only), 2 or 4 (chunk sizes for up to that many codebooks)
template <int V, int NCB>
__global__ __launch_bounds__(kHistThreads, 8) void histogram_kernel(const uint8_t *__restrict__ in,
                                                                 uint64_t seg_n, uint64_t in_stride,
                                                                 uint32_t *__restrict__ partial,
                                                                 const ChunkSizeArgs cs) {
    constexpr uint64_t kPiece = (uint64_t)V * kHistThreads;
    constexpr bool SIZES = NCB != 0;
    __shared__ typename std::conditional<SIZES, SizeSmem, uint4[kHistWords / 4]>::type smem;
    uint4 *hv;
    if constexpr (SIZES) hv = smem.cnt;
    else hv = smem;
    uint32_t *h = reinterpret_cast<uint32_t *>(hv);
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const uint32_t seg = blockIdx.y;
    const uint8_t *base = in + (uint64_t)seg * in_stride;
    // bytes before the first 16-byte boundary, then whole vectors, then a tail
    const uint32_t head_max = (uint32_t)((16 - ((uintptr_t)base & 15)) & 15);
    const uint64_t head = head_max < seg_n ? head_max : seg_n;
    const uint8_t *vbase = base + head;
    const uint64_t n_vec = (seg_n - head) / 16;
    const uint64_t tail = (seg_n - head) % 16;
    const uint4 *vp = reinterpret_cast<const uint4 *>(vbase);

    // the first piece's loads go out before the table is cleared; lanes past
    // the end of the segment (last piece only) load its last vector again and
    // do not count it (unconditional loads keep the waits per load)
    const uint64_t stride = (uint64_t)gridDim.x * kPiece;
    uint64_t p0 = (uint64_t)blockIdx.x * kPiece;
    uint4 q[V];
    auto load = [&](uint64_t p) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint64_t v = p + tid + k * kHistThreads;
            q[k] = vp[v < n_vec ? v : n_vec - 1];
        }
    };
    // counter of byte b in column c: word 32 b + c
    uint32_t *mine = h + (tid & (kHistCols - 1));
    auto count = [&](uint32_t w) __attribute__((always_inline)) {
        atomicAdd(&mine[(w & 0xff) * kHistCols], 1u);
        atomicAdd(&mine[((w >> 8) & 0xff) * kHistCols], 1u);
        atomicAdd(&mine[((w >> 16) & 0xff) * kHistCols], 1u);
        atomicAdd(&mine[(w >> 24) * kHistCols], 1u);
    };
    // with sizes: eight bytes at a time, their length words are read first,
    // then their counters bumped, then the lengths summed into ev
    // (codebooks 0, 2) and od (1, 3), 16 bits each.  A wave's LDS operations
    // complete in order, so waiting for the reads never waits for the
    // counters' atomics issued after them (interleaved, every use would wait
    // for all of them).
    auto count_sized = [&](uint32_t wa, uint32_t wb, uint32_t &ev, uint32_t &od) __attribute__((always_inline)) {
        if constexpr (SIZES) {
            uint32_t e[8], idx[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) idx[j] = (((j < 4 ? wa : wb) >> (8 * (j & 3))) & 0xffu) * kHistCols;
            const uint32_t *lmine = smem.len + (tid & (kHistCols - 1));
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = lmine[idx[j]];
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < 8; ++j) atomicAdd(&mine[idx[j]], 1u);
            asm volatile("" ::: "memory");
            if constexpr (NCB == 2) {
#pragma unroll
                for (int j = 0; j < 8; ++j) ev += e[j];   // codebook 0 in bits 0-7, 1 in bits 16-23
            } else {
                // one byte per codebook: six lengths of at most 40 bits sum
                // within a byte, so bytes are split only twice per eight
                const uint32_t r1 = e[0] + e[1] + e[2] + e[3] + e[4] + e[5], r2 = e[6] + e[7];
                ev += (r1 & 0x00ff00ffu) + (r2 & 0x00ff00ffu);                 // codebooks 0, 2
                od += ((r1 >> 8) & 0x00ff00ffu) + ((r2 >> 8) & 0x00ff00ffu);   // codebooks 1, 3
            }
        }
    };
    // a chunk's share of the sums
    auto add_acc = [&](uint32_t cl, uint32_t ev, uint32_t od) __attribute__((always_inline)) {
        if constexpr (NCB == 2) {
            atomicAdd(&smem.acc[0][cl], ev & 0xffffu);
            if (cs.n_cb > 1) atomicAdd(&smem.acc[1][cl], ev >> 16);
        } else if constexpr (NCB == 4) {
            atomicAdd(&smem.acc[0][cl], ev & 0xffffu);
            if (cs.n_cb > 1) atomicAdd(&smem.acc[1][cl], od & 0xffffu);
            if (cs.n_cb > 2) atomicAdd(&smem.acc[2][cl], ev >> 16);
            if (cs.n_cb > 3) atomicAdd(&smem.acc[3][cl], od >> 16);
        }
    };
    auto count_piece = [&](uint64_t p) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint64_t gv = p + tid + k * kHistThreads;
            if constexpr (!SIZES) {
                if (gv < n_vec) {
                    count(q[k].x);
                    count(q[k].y);
                    count(q[k].z);
                    count(q[k].w);
                }
            } else {
                uint32_t ev = 0, od = 0;
                if (gv < n_vec) {
                    count_sized(q[k].x, q[k].y, ev, od);
                    count_sized(q[k].z, q[k].w, ev, od);
                }
                // this vector's chunk within the piece
                const uint32_t c0 = (uint32_t)(p >> cs.vc_log2);
                if (cs.vc_log2 >= 6) {
                    // the wave's 64 vectors lie in one chunk: the wave adds
                    // its lanes (at most 64 * 16 * 40 bits a half)
                    ev = __builtin_amdgcn_readlane(wave_incl_scan(ev), 63);
                    if constexpr (NCB == 4) od = __builtin_amdgcn_readlane(wave_incl_scan(od), 63);
                    const uint64_t gw = p + wave * 64 + k * kHistThreads;   // the wave's first vector
                    if (lane == 0 && gw < n_vec) add_acc((uint32_t)(gw >> cs.vc_log2) - c0, ev, od);
                } else if (gv < n_vec) {
                    add_acc((uint32_t)(gv >> cs.vc_log2) - c0, ev, od);
                }
            }
        }
    };
    // the piece's chunk sizes, stored once its counts are in (then cleared
    // for the next piece)
    auto store_sizes = [&](uint64_t p) __attribute__((always_inline)) {
        if constexpr (SIZES) {
            __syncthreads();
            const uint32_t cpp = (uint32_t)(kPiece >> cs.vc_log2), c0 = (uint32_t)(p >> cs.vc_log2);
            for (uint32_t t = tid; t < cpp * cs.n_cb; t += kHistThreads) {
                const uint32_t cb = t / cpp, cl = t - cb * cpp;
                if (c0 + cl < cs.chunks_per_seg)
                    cs.sizes[((uint64_t)cb * gridDim.y + seg) * cs.chunks_per_seg + c0 + cl] = (smem.acc[cb][cl] + 127) >> 7;
                smem.acc[cb][cl] = 0;
            }
            __syncthreads();
        }
    };
    const bool any = p0 < n_vec;
    if (any) load(p0);
    for (uint32_t i = tid; i < kHistWords / 4; i += kHistThreads) hv[i] = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (SIZES) {
        // byte b's lengths, one byte per codebook, in every column
        const uint32_t b = tid >> 2;
        uint32_t word = 0;
#pragma unroll
        for (uint32_t cb = 0; cb < (uint32_t)NCB; ++cb)
            if (cb < cs.n_cb) word |= (uint32_t)cs.tabs[cb]->code_len[b] << (8 * cb);
        // two codebooks: the second length moves to bits 16-23, so that a
        // sum over bytes needs no unpacking
        if constexpr (NCB == 2) word = (word & 0xffu) | (word & 0xff00u) << 8;
#pragma unroll
        for (uint32_t c = 0; c < 8; ++c) smem.len[b * kHistCols + 8 * (tid & 3) + c] = word;
        for (uint32_t i = tid; i < kMaxSizeCodebooks * kMaxPieceChunks; i += kHistThreads) (&smem.acc[0][0])[i] = 0;
    }
    __syncthreads();
    if (any) {
        count_piece(p0);
        store_sizes(p0);
        for (p0 += stride; p0 < n_vec; p0 += stride) {
            load(p0);
            count_piece(p0);
            store_sizes(p0);
        }
    }
    if (blockIdx.x == 0 && tid < head) atomicAdd(&mine[base[tid] * kHistCols], 1u);
    if (blockIdx.x == 0 && tid < tail) atomicAdd(&mine[vbase[n_vec * 16 + tid] * kHistCols], 1u);
    __syncthreads();

    // thread t sums eight columns of bin t >> 2 (quarter t & 3), rotated by
    // the bin so that the 32 lanes of one pass read 32 different banks; the
    // four quarters are then added across lanes
    const uint32_t bin = tid >> 2, qtr = tid & 3;
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += h[bin * kHistCols + qtr * 8 + ((j + bin) & 7)];
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    if (qtr == 0) partial[((uint64_t)seg * 256 + bin) * gridDim.x + blockIdx.x] = sum;   // bin-major rows
}

// Workgroup (bin, seg), one wave: lane l adds the partial counts of rows
// l, l + 64, ... (contiguous in the bin-major layout, eight loads in
// flight), then the wave adds its lanes.
__global__ __launch_bounds__(64) void histogram_reduce_kernel(const uint32_t *__restrict__ partial, uint32_t rows,
                                                              uint64_t *__restrict__ counts) {
    const uint32_t l = threadIdx.x;
    const uint64_t bin = (uint64_t)blockIdx.y * 256 + blockIdx.x;
    const uint32_t *src = partial + bin * rows;
    uint64_t s0 = 0, s1 = 0;
    uint32_t r = l;
    for (; r + 7 * 64 < rows; r += 8 * 64) {
        uint32_t x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = src[r + k * 64];
        s0 += ((uint64_t)x[0] + x[1]) + ((uint64_t)x[2] + x[3]);
        s1 += ((uint64_t)x[4] + x[5]) + ((uint64_t)x[6] + x[7]);
    }
    for (; r < rows; r += 64) s0 += src[r];
    uint64_t v = s0 + s1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if (l == 0) counts[bin] = v;
}

// ------------------------------------------------------------ PMF average

// Block reduction of a 64-bit value over 256 threads (fixed order).
__device__ uint64_t block_sum_u64(uint64_t v, uint64_t *scratch) {
    const uint32_t tid = threadIdx.x;
    scratch[tid] = v;
    __syncthreads();
    for (uint32_t s = 128; s > 0; s >>= 1) {
        if (tid < s) scratch[tid] += scratch[tid + s];
        __syncthreads();
    }
    uint64_t r = scratch[0];
    __syncthreads();
    return r;
}

// d_pmf[b] = mean over rows of counts[row][b] / total(row), fp32 with a
// compensated (Kahan) running sum over the rows.
__global__ __launch_bounds__(256) void pmf_average_kernel(const uint64_t *__restrict__ counts,
                                                          uint32_t n_seg, float *__restrict__ pmf) {
    __shared__ uint64_t scratch[256];
    const uint32_t b = threadIdx.x;
    float sum = 0.f, comp = 0.f;
    for (uint32_t s = 0; s < n_seg; ++s) {
        uint64_t c = counts[(uint64_t)s * 256 + b];
        uint64_t total = block_sum_u64(c, scratch);
        if (total == 0) continue;
        float p = (float)c / (float)total;
        float y = p - comp;
        float t = sum + y;
        comp = (t - sum) - y;
        sum = t;
    }
    pmf[b] = n_seg ? sum / (float)n_seg : 0.f;
}

// ------------------------------------------------------------------ KL

// phi(d) = (1 + d) ln(1 + d) - d >= 0, the Bregman term of KL in the ratio
// r = 1 + d.  A series for small |d| avoids the cancellation of the closed
// form: phi(d) = sum_{j>=2} (-1)^j d^j / (j (j - 1)).
__device__ float kl_phi(float d) {
    if (d <= -1.f) return 1.f;
    if (fabsf(d) < 0.25f) {
        float acc = 0.f;
#pragma unroll
        for (int j = 14; j >= 3; --j) acc = 1.f / (float)(j * (j - 1)) - d * acc;
        // acc = 1/6 - d/12 + d^2/20 - ... ; phi = d^2 (1/2 - d * acc)
        return d * d * (0.5f - d * acc);
    }
    return (1.f + d) * log1pf(d) - d;
}

// Sum of a 64-bit value over the 256 threads of a workgroup: DPP-free wave
// reduction with cross-lane adds, then the four wave totals through LDS.
__device__ __forceinline__ uint64_t wg_sum_u64(uint64_t v, uint64_t *w4) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if ((threadIdx.x & 63) == 0) w4[threadIdx.x >> 6] = v;
    __syncthreads();
    return w4[0] + w4[1] + w4[2] + w4[3];
}
__device__ __forceinline__ float wg_sum_f32(float v, float *w4) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if ((threadIdx.x & 63) == 0) w4[threadIdx.x >> 6] = v;
    __syncthreads();
    return (w4[0] + w4[1]) + (w4[2] + w4[3]);
}

// One workgroup per row: D(P_row || Q) = sum_b Q_b phi(P_b / Q_b - 1) / ln 2,
// which equals sum P log2(P / Q) because both distributions sum to one.
// d = (p Nq - q Np) / (q Np) comes from exact integer products.
__global__ __launch_bounds__(256) void pmf_kl_kernel(const uint64_t *__restrict__ pc, uint32_t n_seg,
                                                     const uint64_t *__restrict__ qc, uint32_t q_add,
                                                     float *__restrict__ kl) {
    __shared__ uint64_t w_np[4], w_nq[4];
    __shared__ float w_t[4];
    __shared__ int any_inf;
    const uint32_t b = threadIdx.x;
    const uint32_t row = blockIdx.x;
    if (b == 0) any_inf = 0;
    const uint64_t p = pc[(uint64_t)row * 256 + b];
    const uint64_t q = qc[b] + q_add;
    const uint64_t np = wg_sum_u64(p, w_np);
    const uint64_t nq = wg_sum_u64(q, w_nq);
    float term;
    bool inf = false;
    if (np == 0) {
        term = 0.f;
    } else if (q == 0) {
        term = 0.f;
        inf = p > 0;
    } else if (p == 0) {
        term = (float)q / (float)nq;               // phi(-1) = 1
    } else {
        float d;
        if (np < (1ull << 31) && nq < (1ull << 31)) {
            int64_t num = (int64_t)(p * nq) - (int64_t)(q * np);
            uint64_t den = q * np;
            d = (float)num / (float)den;
        } else {
            double r = ((double)p * (double)nq) / ((double)q * (double)np);
            d = (float)(r - 1.0);
        }
        term = ((float)q / (float)nq) * kl_phi(d);
    }
    if (inf) any_inf = 1;
    const float sum = wg_sum_f32(term, w_t);
    if (b == 0) kl[row] = any_inf ? __builtin_inff() : sum * 1.4426950408889634f;  // 1 / ln 2
}

}  // namespace

// Workgroups per segment: one per piece of the segment (128 KiB, 64 KiB with
// chunk sizes, or 16 KiB when the whole launch has fewer than 256 pieces of
// 128 KiB), at most
// 4096 rows of partial counts over all segments (but at least one per
// segment); a workgroup then takes every gridDim.x-th piece of its segment.
// A workgroup reads at most max(seg_n, n_seg * seg_n / 4096) bytes plus a
// piece (2^28 for the largest accepted segment), a 32-bit partial count
// holds that, and one counter sees a 1/32 share of it.
static bool histogram_small(uint64_t seg_n, uint32_t n_seg) {
    return (seg_n / 16 + kHistPiece - 1) / kHistPiece * n_seg < 256;
}

bool histogram_can_size(uint64_t seg_n, uint32_t n_seg, uint32_t chunk_symbols) {
    const uint64_t piece_bytes = 16 * (histogram_small(seg_n, n_seg) ? (uint64_t)kHistThreads : kSizedPiece);
    return chunk_symbols >= 256 && (chunk_symbols & (chunk_symbols - 1)) == 0 && piece_bytes % chunk_symbols == 0 &&
           seg_n % 16 == 0;
}

uint32_t histogram_blocks(uint64_t seg_n, uint32_t n_seg, bool sized) {
    const uint64_t piece = histogram_small(seg_n, n_seg) ? kHistThreads : sized ? kSizedPiece : kHistPiece;
    uint64_t blocks = (seg_n / 16 + piece - 1) / piece;
    const uint64_t cap = n_seg < 4096 ? 4096 / n_seg : 1;
    if (blocks > cap) blocks = cap;
    return blocks ? (uint32_t)blocks : 1u;
}

hipError_t launch_histogram(const uint8_t *in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride,
                            uint64_t *counts, uint32_t *partial, const ChunkSizeArgs *cs, hipStream_t s) {
    const uint32_t blocks = histogram_blocks(seg_n, n_seg, cs != nullptr);
    const ChunkSizeArgs none = {};
    const bool small = histogram_small(seg_n, n_seg);
    const dim3 grid(blocks, n_seg), wg(kHistThreads);
    if (cs && cs->n_cb <= 2) {
        if (small) hipLaunchKernelGGL((histogram_kernel<1, 2>), grid, wg, 0, s, in, seg_n, in_stride, partial, *cs);
        else hipLaunchKernelGGL((histogram_kernel<kHistVecSized, 2>), grid, wg, 0, s, in, seg_n, in_stride, partial, *cs);
    } else if (cs) {
        if (small) hipLaunchKernelGGL((histogram_kernel<1, 4>), grid, wg, 0, s, in, seg_n, in_stride, partial, *cs);
        else hipLaunchKernelGGL((histogram_kernel<kHistVecSized, 4>), grid, wg, 0, s, in, seg_n, in_stride, partial, *cs);
    } else if (small) {
        hipLaunchKernelGGL((histogram_kernel<1, 0>), grid, wg, 0, s, in, seg_n, in_stride, partial, none);
    } else {
        hipLaunchKernelGGL((histogram_kernel<kHistVec, 0>), grid, wg, 0, s, in, seg_n, in_stride, partial, none);
    }
    hipLaunchKernelGGL(histogram_reduce_kernel, dim3(256, n_seg), dim3(64), 0, s, partial, blocks, counts);
    return hipGetLastError();
}

hipError_t launch_pmf_average(const uint64_t *counts, uint32_t n_seg, float *pmf, hipStream_t s) {
    hipLaunchKernelGGL(pmf_average_kernel, dim3(1), dim3(256), 0, s, counts, n_seg, pmf);
    return hipGetLastError();
}

hipError_t launch_pmf_kl(const uint64_t *p, uint32_t n_seg, const uint64_t *q, uint32_t q_add, float *kl,
                         hipStream_t s) {
    if (n_seg == 0) return hipSuccess;
    hipLaunchKernelGGL(pmf_kl_kernel, dim3(n_seg), dim3(256), 0, s, p, n_seg, q, q_add, kl);
    return hipGetLastError();
}

}  // namespace ec
