// Byte histogram and the PMF statistics kernels.
//
// Histogram, two launches:
//   1. histogram_kernel: each workgroup counts a contiguous slice of one
//      segment into LDS bins privatised per wave and per lane group (so the
//      skewed e4m3 distributions, where a few bytes dominate, do not
//      serialise the LDS atomics), then stores its 256 partial counts with
//      plain stores;
//   2. histogram_reduce_kernel: sums the partial rows of each segment into
//      the 64-bit counts, a slice of 16 bins per workgroup.
// No global atomics: same-address atomics from many workgroups serialise at
// the memory side.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kHistThreads = 256;
constexpr int kHistCopies = 8;                 // LDS copies per wave (lane & 7)
constexpr int kHistStride = 257;               // words per copy: copies of one bin fall in different banks
constexpr int kHistVecPerThread = 16;          // 16-byte loads per thread per block (64 KiB per block)
constexpr int kReduceBins = 2;                 // bins per reduce workgroup
constexpr int kReduceGroups = 256 / kReduceBins;

__global__ __launch_bounds__(kHistThreads) void histogram_kernel(const uint8_t *__restrict__ in,
                                                                 uint64_t seg_n, uint64_t in_stride,
                                                                 uint64_t vec_per_block,
                                                                 uint32_t *__restrict__ partial) {
    constexpr int kCopies = kHistThreads / 64 * kHistCopies;
    __shared__ uint32_t bins[kCopies * kHistStride];
    const uint32_t tid = threadIdx.x;
    uint32_t *mine = bins + ((tid >> 6) * kHistCopies + (tid & (kHistCopies - 1))) * kHistStride;
    for (uint32_t i = tid; i < kCopies * kHistStride; i += kHistThreads) bins[i] = 0;
    __syncthreads();

    const uint32_t seg = blockIdx.y;
    const uint8_t *base = in + (uint64_t)seg * in_stride;
    // bytes before the first 16-byte boundary, then whole vectors, then a tail
    const uint32_t head_max = (uint32_t)((16 - ((uintptr_t)base & 15)) & 15);
    const uint64_t head = head_max < seg_n ? head_max : seg_n;
    const uint8_t *vbase = base + head;
    const uint64_t n_vec = (seg_n - head) / 16;
    const uint64_t tail = (seg_n - head) % 16;
    const uint64_t v0 = (uint64_t)blockIdx.x * vec_per_block;
    const uint64_t v1 = v0 + vec_per_block < n_vec ? v0 + vec_per_block : n_vec;
    const uint4 *vp = reinterpret_cast<const uint4 *>(vbase);
    auto count = [&](const uint4 &q) __attribute__((always_inline)) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&mine[w[k] & 0xff], 1u);
            atomicAdd(&mine[(w[k] >> 8) & 0xff], 1u);
            atomicAdd(&mine[(w[k] >> 16) & 0xff], 1u);
            atomicAdd(&mine[w[k] >> 24], 1u);
        }
    };
    // four vectors in flight per thread
    uint64_t v = v0 + tid;
    for (; v + 3 * kHistThreads < v1; v += 4 * kHistThreads) {
        const uint4 q0 = vp[v], q1 = vp[v + kHistThreads], q2 = vp[v + 2 * kHistThreads], q3 = vp[v + 3 * kHistThreads];
        count(q0);
        count(q1);
        count(q2);
        count(q3);
    }
    for (; v < v1; v += kHistThreads) count(vp[v]);
    if (blockIdx.x == 0 && tid < head) atomicAdd(&mine[base[tid]], 1u);
    if (blockIdx.x == 0 && tid < tail) atomicAdd(&mine[vbase[n_vec * 16 + tid]], 1u);
    __syncthreads();

    uint32_t sum = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) sum += bins[c * kHistStride + tid];
    partial[((uint64_t)seg * gridDim.x + blockIdx.x) * 256 + tid] = sum;
}

// Workgroup (j, seg) sums bins [2 j, 2 j + 2) of segment seg over its `rows`
// partial rows: thread t takes bin t % 2 and every 128th row from t / 2
// (eight loads in flight), then the 128 row groups are added in LDS.
__global__ __launch_bounds__(256) void histogram_reduce_kernel(const uint32_t *__restrict__ partial, uint32_t rows,
                                                               uint64_t *__restrict__ counts) {
    __shared__ uint64_t acc[kReduceGroups][kReduceBins];
    const uint32_t tid = threadIdx.x, b = tid % kReduceBins, g = tid / kReduceBins;
    const uint32_t bin = blockIdx.x * kReduceBins + b;
    const uint32_t *src = partial + (uint64_t)blockIdx.y * rows * 256 + bin;
    uint64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    uint32_t r = g;
    for (; r + 7 * kReduceGroups < rows; r += 8 * kReduceGroups) {
        uint32_t x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = src[(uint64_t)(r + k * kReduceGroups) * 256];
        s0 += (uint64_t)x[0] + x[1];
        s1 += (uint64_t)x[2] + x[3];
        s2 += (uint64_t)x[4] + x[5];
        s3 += (uint64_t)x[6] + x[7];
    }
    for (; r < rows; r += kReduceGroups) s0 += src[(uint64_t)r * 256];
    acc[g][b] = s0 + s1 + s2 + s3;
    __syncthreads();
    for (uint32_t h = kReduceGroups / 2; h > 0; h >>= 1) {
        if (g < h) acc[g][b] += acc[g + h][b];
        __syncthreads();
    }
    if (g == 0) counts[(uint64_t)blockIdx.y * 256 + bin] = acc[0][b];
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

// Workgroups per segment: one per 4096 16-byte vectors, at most 65536 rows
// of partial counts over all segments (but at least one per segment).
uint32_t histogram_blocks(uint64_t seg_n, uint32_t n_seg) {
    const uint64_t n_vec = seg_n / 16;
    const uint64_t per_block = (uint64_t)kHistThreads * kHistVecPerThread;
    uint64_t blocks = (n_vec + per_block - 1) / per_block;
    const uint64_t cap = n_seg < 65536 ? 65536 / n_seg : 1;
    if (blocks > cap) blocks = cap;
    return blocks ? (uint32_t)blocks : 1u;
}

hipError_t launch_histogram(const uint8_t *in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride,
                            uint64_t *counts, uint32_t *partial, hipStream_t s) {
    const uint32_t blocks = histogram_blocks(seg_n, n_seg);
    const uint64_t n_vec = seg_n / 16;
    const uint64_t per_block = (n_vec + blocks - 1) / blocks;
    hipLaunchKernelGGL(histogram_kernel, dim3(blocks, n_seg), dim3(kHistThreads), 0, s, in, seg_n, in_stride,
                       per_block, partial);
    hipLaunchKernelGGL(histogram_reduce_kernel, dim3(256 / kReduceBins, n_seg), dim3(256), 0, s, partial, blocks,
                       counts);
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
