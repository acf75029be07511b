// Byte histogram and the PMF statistics kernels.
//
// Histogram, two launches:
//   1. histogram_kernel: the workgroups of a segment sweep it together in
//      rounds of 32 KiB per workgroup, counting into LDS counters; each then
//      stores its 256 partial counts with plain stores.  Every wave owns 16 columns of 256 counters; lane l adds
//      into column l & 15, so the counter of byte b is word 16 b + (l & 15):
//      whatever bytes the 32 lanes of one LDS pass hold, at most two of them
//      share a bank (random addresses into one shared table, and the skewed
//      e4m3 distributions where a few bytes dominate, cost several times
//      more);
//   2. histogram_reduce_kernel: sums the partial rows of each segment into
//      the 64-bit counts, one wave per bin.
// No global atomics: same-address atomics from many workgroups serialise at
// the memory side.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kHistThreads = 256;
constexpr int kHistCols = 16;                          // counter columns per wave (lane & 15)
constexpr int kHistWaveWords = 256 * kHistCols;        // 16 KiB of counters per wave
constexpr int kHistRoundVec = 8;                       // 16-byte loads in flight per thread per round
constexpr uint64_t kHistRound = (uint64_t)kHistRoundVec * kHistThreads;   // vectors per workgroup round
constexpr int kHistRoundsPerBlock = 4;                 // target rounds per workgroup (128 KiB)

__global__ __launch_bounds__(kHistThreads) void histogram_kernel(const uint8_t *__restrict__ in,
                                                                 uint64_t seg_n, uint64_t in_stride,
                                                                 uint32_t *__restrict__ partial) {
    constexpr int kWaves = kHistThreads / 64;
    __shared__ uint4 hv[kWaves * kHistWaveWords / 4];
    uint32_t *h = reinterpret_cast<uint32_t *>(hv);
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (uint32_t i = tid; i < kWaves * kHistWaveWords / 4; i += kHistThreads) hv[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    // a word takes the bytes of 4 lanes of one workgroup: far below 2^32
    uint32_t *mine = h + wave * kHistWaveWords + (lane & (kHistCols - 1));

    const uint32_t seg = blockIdx.y;
    const uint8_t *base = in + (uint64_t)seg * in_stride;
    // bytes before the first 16-byte boundary, then whole vectors, then a tail
    const uint32_t head_max = (uint32_t)((16 - ((uintptr_t)base & 15)) & 15);
    const uint64_t head = head_max < seg_n ? head_max : seg_n;
    const uint8_t *vbase = base + head;
    const uint64_t n_vec = (seg_n - head) / 16;
    const uint64_t tail = (seg_n - head) % 16;
    const uint4 *vp = reinterpret_cast<const uint4 *>(vbase);
    auto count = [&](const uint4 &q) __attribute__((always_inline)) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&mine[(w[k] & 0xff) * kHistCols], 1u);
            atomicAdd(&mine[((w[k] >> 8) & 0xff) * kHistCols], 1u);
            atomicAdd(&mine[((w[k] >> 16) & 0xff) * kHistCols], 1u);
            atomicAdd(&mine[(w[k] >> 24) * kHistCols], 1u);
        }
    };
    // grid-stride rounds: at any time the workgroups of a segment read one
    // contiguous window of it; every load of a round is issued before its
    // first count, and each count waits for its own load only
    for (uint64_t r0 = (uint64_t)blockIdx.x * kHistRound; r0 < n_vec; r0 += (uint64_t)gridDim.x * kHistRound) {
        const uint64_t v = r0 + tid;
        uint4 q[kHistRoundVec];
        if (r0 + kHistRound <= n_vec) {
#pragma unroll
            for (int k = 0; k < kHistRoundVec; ++k) q[k] = vp[v + k * kHistThreads];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < kHistRoundVec; ++k) count(q[k]);
        } else {   // the segment's last, partial round
#pragma unroll
            for (int k = 0; k < kHistRoundVec; ++k) {
                if (v + k * kHistThreads < n_vec) q[k] = vp[v + k * kHistThreads];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < kHistRoundVec; ++k) {
                if (v + k * kHistThreads < n_vec) count(q[k]);
            }
        }
    }
    if (blockIdx.x == 0 && tid < head) atomicAdd(&mine[base[tid] * kHistCols], 1u);
    if (blockIdx.x == 0 && tid < tail) atomicAdd(&mine[vbase[n_vec * 16 + tid] * kHistCols], 1u);
    __syncthreads();

    // thread t sums byte t over all columns, starting at column t & 15 so
    // that the lanes of one access spread over the banks
    uint32_t sum = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
#pragma unroll
        for (int j = 0; j < kHistCols; ++j) sum += h[w * kHistWaveWords + tid * kHistCols + ((j + tid) & (kHistCols - 1))];
    }
    partial[((uint64_t)seg * 256 + tid) * gridDim.x + blockIdx.x] = sum;   // bin-major rows
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

// Workgroups per segment: one per kHistRoundsPerBlock rounds of the
// segment, at most 65536 rows of partial counts over all segments (but at
// least one per segment).
uint32_t histogram_blocks(uint64_t seg_n, uint32_t n_seg) {
    const uint64_t rounds = (seg_n / 16 + kHistRound - 1) / kHistRound;
    uint64_t blocks = (rounds + kHistRoundsPerBlock - 1) / kHistRoundsPerBlock;
    const uint64_t cap = n_seg < 65536 ? 65536 / n_seg : 1;
    if (blocks > cap) blocks = cap;
    return blocks ? (uint32_t)blocks : 1u;
}

hipError_t launch_histogram(const uint8_t *in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride,
                            uint64_t *counts, uint32_t *partial, hipStream_t s) {
    const uint32_t blocks = histogram_blocks(seg_n, n_seg);
    hipLaunchKernelGGL(histogram_kernel, dim3(blocks, n_seg), dim3(kHistThreads), 0, s, in, seg_n, in_stride,
                       partial);
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
