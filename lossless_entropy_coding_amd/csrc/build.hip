// Per-shard Huffman codebooks built on the GPU: the codebook-generation stage
// of the three-stage design ("Single-Stage Huffman Encoder for ML
// Compression", abstract: frequency analysis, codebook generation and
// transmission, encoding), so that a batch of shards goes from histogram rows
// to encoded streams without a trip through host memory.
//
// One workgroup of 256 threads builds the tables of one shard, bit for bit
// the tables the host builder makes from the same counts:
//   1. weights counts[b] + 1; the leaves in stable order of weight (the rank
//      of (weight, byte) among all 256, counted by every thread for its byte);
//   2. the two-queue merge (leaves in sorted order, merged nodes in creation
//      order; the lighter front is taken, the leaf on a tie), run by one wave
//      with uniform scalar control flow, the four candidate fronts of a step
//      read from LDS together;
//   3. every node's depth by pointer jumping over the parent links (nine
//      rounds cover the deepest possible tree of 256 leaves);
//   4. canonical codes: the number of codes of each length, the first code
//      and first canonical position of each length, each byte's position in
//      (length, byte) order;
//   5. the tables: left-aligned encode entries, the 13-bit decode table (a
//      window's code length is one more than the number of 13-bit limits at
//      or below it), the 40-bit canonical limits, the canonical symbol order,
//      the code lengths and the FNV-1a codebook id.
// The same steps 4 and 5 also rebuild a codebook from the code lengths a
// stream carries (huff_tables_from_streams_kernel).
// A code longer than EC_MAX_CODE_LEN bits, or a count of 2^55 or more, makes
// the shard's table unusable (codec 0, all entries zero) and sets
// EC_S_BAD_CODEBOOK in its status word.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kBuildThreads = 256;
constexpr uint32_t kNodes = 511;                 // 256 leaves + 255 merged nodes
constexpr uint32_t kRoot = 510;
constexpr uint64_t kHeavy = ~0ull;               // weight of an empty queue front
constexpr uint64_t kMaxCount = 1ull << 55;       // larger counts could overflow the 64-bit node weights

struct BuildSmem {
    uint64_t w[256];          // weight by byte; later the code length by byte, as a 64-bit key
    uint64_t sw[256 + 2];     // leaf weights in sorted order (+2 heavy sentinels)
    uint64_t iw[256 + 2];     // merged-node weights in creation order
    uint32_t sw32[256 + 4];   // the same as 32-bit weights (small shards), +4 heavy sentinels
    uint32_t iw32[256 + 4];
    uint64_t fcode[48];       // first canonical code of each length
    uint32_t fidx[48];        // first canonical position of each length
    uint32_t blc[64];         // codes of each length
    uint32_t lim13[16];       // end of the codes of length l as 13-bit windows
    uint16_t par[512];        // parent of node v (leaf at sorted position p: v = p; merged node k: 256 + k)
    uint16_t anc[512];        // pointer-jumping ancestor
    uint16_t dep[512];        // distance from v to anc[v]
    uint8_t sidx[256];        // byte at sorted position
    uint8_t len[256];         // code length by byte
    uint8_t symc[256];        // byte at canonical position
    uint32_t bad, max_len, wide;
};

// Rank of (key[s], s) among the 256 pairs (key[j], j) in lexicographic
// order: the number of pairs below it.  Every thread counts for its own s
// over the same broadcast LDS reads.
__device__ __forceinline__ uint32_t rank256(const uint64_t *key, uint64_t ks, uint32_t s) {
    uint32_t r = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < 256; ++j) {
        const uint64_t kj = key[j];
        r += (kj < ks || (kj == ks && j < s)) ? 1u : 0u;
    }
    return r;
}

__device__ __forceinline__ uint32_t rank256_32(const uint32_t *key, uint32_t ks, uint32_t s) {
    uint32_t r = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < 256; ++j) {
        const uint32_t kj = key[j];
        r += (kj < ks || (kj == ks && j < s)) ? 1u : 0u;
    }
    return r;
}

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (uint64_t)hi << 32 | lo;
}

// An unusable table (codec 0, every entry zero), and the status bits saying why.
__device__ void unusable_table(DevTables *t, uint32_t tid, uint32_t *status, uint32_t bits) {
    uint4 *p = reinterpret_cast<uint4 *>(t);
    for (uint32_t i = tid; i < sizeof(DevTables) / 16; i += kBuildThreads) p[i] = make_uint4(0, 0, 0, 0);
    if (tid == 0) or_status(status, bits);
}

// Steps 4 and 5, from the code lengths in sm.len (a complete code, every
// length 1..EC_MAX_CODE_LEN), their counts sm.blc and sm.max_len.  Called
// by every thread of the workgroup.
__device__ void canonical_tables(BuildSmem &sm, DevTables *t, uint32_t tid) {
    const uint32_t wave = tid >> 6;
    // 4. canonical codes.  first_code[l] = sum_{j<l} blc[j] << (l - j) and
    // first_idx[l] = sum_{j<l} blc[j] (the recurrence c_l = (c_{l-1} +
    // blc[l-1]) << 1 unrolled).
    if (tid < 48) {
        uint64_t fc = 0;
        uint32_t fi = 0;
        if (tid >= 1 && tid <= (uint32_t)EC_MAX_CODE_LEN) {
            for (uint32_t j = 1; j < tid; ++j) {
                fc += (uint64_t)sm.blc[j] << (tid - j);
                fi += sm.blc[j];
            }
        }
        sm.fcode[tid] = fc;
        sm.fidx[tid] = fi;
    }
    const uint32_t my_len = sm.len[tid];
    sm.w[tid] = my_len;   // (length, byte) keys for the canonical order
    __syncthreads();
    if (tid >= 1 && tid <= (uint32_t)kHuffBits)
        sm.lim13[tid] = (uint32_t)((sm.fcode[tid] + sm.blc[tid]) << (kHuffBits - tid));
    const uint32_t pos = rank256(sm.w, my_len, tid);
    sm.symc[pos] = (uint8_t)tid;
    const uint64_t code = sm.fcode[my_len] + (pos - sm.fidx[my_len]);
    const uint32_t max_len = sm.max_len;
    __syncthreads();

    // 5. tables
    t->enc64[tid] = (code << (64 - my_len)) | my_len;
    t->enc32[tid] = max_len <= (uint32_t)kNarrowMaxLen ? ((uint32_t)code << (32 - my_len)) | my_len : 0u;
    t->sym[tid] = sm.symc[tid];
    t->code_len[tid] = (uint8_t)my_len;
    for (uint32_t i = tid; i < (uint32_t)kL1Size; i += kBuildThreads) t->l1[i] = 0;
    if (tid < 48) {
        const bool in = tid >= 1 && tid <= (uint32_t)EC_MAX_CODE_LEN;
        t->limit[tid] = in ? (sm.fcode[tid] + sm.blc[tid]) << (EC_MAX_CODE_LEN - tid) : 0ull;
        t->first_code[tid] = in ? sm.fcode[tid] : 0ull;
        t->first_idx[tid] = in ? sm.fidx[tid] : 0u;
    }
    if (wave == 0) {
        // codebook id: FNV-1a 64 over the codec byte and the 256 code lengths
        if (tid == 0) {
            uint64_t h = 0xcbf29ce484222325ull;
            h = (h ^ (uint64_t)EC_CODEC_HUFFMAN) * 0x100000001b3ull;
            for (uint32_t s = 0; s < 256; ++s) h = (h ^ (uint64_t)sm.len[s]) * 0x100000001b3ull;
            t->codebook_id = h;
            t->codec = EC_CODEC_HUFFMAN;
            t->max_len = max_len;
            t->qlc_lens = 0;
            t->eg_k = -1;
            t->pad[0] = 0;
            t->pad[1] = 0;
        }
    } else {
        // 13-bit decode table: window w starts a code of length
        // l = 1 + #{l' <= 13 : lim13[l'] <= w}; none when l > 13
        uint32_t lim[kHuffBits + 1];
#pragma unroll
        for (int l = 1; l <= kHuffBits; ++l) lim[l] = sm.lim13[l];
        for (uint32_t w = tid - 64; w < (uint32_t)kHuffSize; w += kBuildThreads - 64) {
            uint32_t l = 1;
#pragma unroll
            for (int j = 1; j <= kHuffBits; ++j) l += lim[j] <= w ? 1u : 0u;
            uint16_t e = 0;
            if (l <= (uint32_t)kHuffBits) {
                const uint32_t idx = sm.fidx[l] + (uint32_t)((w >> (kHuffBits - l)) - sm.fcode[l]);
                e = (uint16_t)(l | ((uint32_t)sm.symc[idx & 255u] << 8));
            }
            t->hl1[w] = e;
        }
    }
}

// Step 2 for weights that fit 32 bits, in as few scalar instructions a step
// as the merge allows (one wave issues an instruction at most every few
// cycles, so the step's length is its instruction count): the fronts of
// both queues (L0 L1, Q0 Q1) stay in scalar registers, and the entries
// that may become fronts next (leaves li + 2, li + 3; merged nodes qh + 2,
// qh + 3) are read at the start of each step and taken up at its end.  A
// merged node at or past qt reads as heavy, the one made in the step as its
// sum.  Same takes as the 64-bit loop: the lighter front, the leaf on a tie.
__device__ __forceinline__ uint32_t rfl(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ void merge32(BuildSmem &sm) {
    constexpr uint32_t H = 0xffffffffu;
    uint32_t li = 0, qh = 0, qt = 0;
    uint32_t L0 = rfl(sm.sw32[0]), L1 = rfl(sm.sw32[1]), Q0 = H, Q1 = H;
#pragma unroll 3
    for (uint32_t k = 0; k < 255; ++k) {
        const uint32_t l2 = sm.sw32[li + 2], l3 = sm.sw32[li + 3];
        const uint32_t q2 = sm.iw32[qh + 2], q3 = sm.iw32[qh + 3];
        uint32_t id0, id1, sum, cl, cq;
        if (L0 <= Q0) {
            if (L1 <= Q0) {
                id0 = li;
                id1 = li + 1;
                sum = L0 + L1;
                cl = 2;
                cq = 0;
            } else {
                id0 = li;
                id1 = 256 + qh;
                sum = L0 + Q0;
                cl = 1;
                cq = 1;
            }
        } else if (L0 <= Q1) {
            id0 = 256 + qh;
            id1 = li;
            sum = Q0 + L0;
            cl = 1;
            cq = 1;
        } else {
            id0 = 256 + qh;
            id1 = 256 + qh + 1;
            sum = Q0 + Q1;
            cl = 0;
            cq = 2;
        }
        // every lane writes the same values (no branch on the lane)
        sm.iw32[qt] = sum;
        sm.par[id0] = (uint16_t)(256 + qt);
        sm.par[id1] = (uint16_t)(256 + qt);
        // leaf fronts
        const uint32_t L2 = rfl(l2), L3 = rfl(l3);
        if (cl == 1) {
            L0 = L1;
            L1 = L2;
        } else if (cl == 2) {
            L0 = L2;
            L1 = L3;
        }
        // merged-node fronts at qh + cq and qh + cq + 1 (node qt is new)
        const uint32_t Q2 = rfl(q2), Q3 = rfl(q3);
        const uint32_t a = cq, b = cq + 1;   // window offsets, 0..3
        const uint32_t va = a == 0 ? Q0 : a == 1 ? Q1 : Q2;
        const uint32_t vb = b == 1 ? Q1 : b == 2 ? Q2 : Q3;
        const uint32_t pa = qh + a, pb = qh + b;
        Q0 = pa < qt ? va : pa == qt ? sum : H;
        Q1 = pb < qt ? vb : pb == qt ? sum : H;
        li += cl;
        qh += cq;
        ++qt;
    }
}

__global__ __launch_bounds__(kBuildThreads) void huff_build_kernel(const uint64_t *counts, DevTables *tabs,
                                                                   uint32_t *status) {
    __shared__ BuildSmem sm;
    const uint32_t tid = threadIdx.x, wave = tid >> 6;
    const uint32_t seg = blockIdx.x;
    DevTables *t = tabs + seg;

    // 1. weights and the stable sort of the leaves
    const uint64_t c = counts[(uint64_t)seg * 256 + tid];
    const uint64_t ws = c + 1;
    if (tid == 0) {
        sm.bad = 0;
        sm.max_len = 0;
        sm.wide = 0;
    }
    if (tid < 64) sm.blc[tid] = 0;
    sm.w[tid] = ws;
    __syncthreads();
    if (c >= kMaxCount) sm.bad = 1;
    // counts below 2^23 keep every node weight (at most 256 * 2^23) in 32 bits
    if (c >= (1ull << 23)) sm.wide = 1;
    __syncthreads();   // sm.wide settled
    uint32_t r;
    if (!sm.wide) {
        // 32-bit keys (count + 1 below 2^23 + 1): half the compares
        uint32_t *k32 = reinterpret_cast<uint32_t *>(sm.iw32);   // scratch until the merge
        k32[tid] = (uint32_t)ws;
        __syncthreads();
        r = rank256_32(k32, (uint32_t)ws, tid);
        __syncthreads();   // the keys are read by all before iw32 is reused
    } else {
        r = rank256(sm.w, ws, tid);
    }
    sm.sw[r] = ws;
    sm.sw32[r] = (uint32_t)ws;
    sm.sidx[r] = (uint8_t)tid;
    if (tid < 4) {
        sm.sw32[256 + tid] = 0xffffffffu;
        sm.iw32[256 + tid] = 0xffffffffu;
    }
    if (tid < 2) {
        sm.sw[256 + tid] = kHeavy;
        sm.iw[256 + tid] = kHeavy;
    }
    __syncthreads();

    // 2. two-queue merge, one wave; li / qh / qt and the fronts are uniform.
    // A step takes two nodes, so the two leading entries of each queue are
    // all it can need: they are read together at the start of the step.
    // Every take finds a node in one of the queues (a step starts with at
    // least two), so li <= 256 and qh < qt whatever the weights.
    if (wave == 0 && !sm.wide) {
        merge32(sm);
        sm.par[kRoot] = (uint16_t)kRoot;
    } else if (wave == 0) {
        uint32_t li = 0, qh = 0, qt = 0;
        for (uint32_t k = 0; k < 255; ++k) {
            uint64_t l0 = uniform64(sm.sw[li]), l1 = uniform64(sm.sw[li + 1]);
            uint64_t q0 = qh < qt ? uniform64(sm.iw[qh]) : kHeavy;
            uint64_t q1 = qh + 1 < qt ? uniform64(sm.iw[qh + 1]) : kHeavy;
            uint32_t id[2];
            uint64_t wt[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (li < 256 && l0 <= q0) {   // the leaf on a tie
                    id[m] = li++;
                    wt[m] = l0;
                    l0 = l1;
                } else {
                    id[m] = 256 + qh++;
                    wt[m] = q0;
                    q0 = q1;
                }
            }
            const uint64_t sum = wt[0] + wt[1];
            if (tid == 0) {
                sm.iw[qt] = sum;
                sm.par[id[0]] = (uint16_t)(256 + qt);
                sm.par[id[1]] = (uint16_t)(256 + qt);
            }
            ++qt;
        }
        if (tid == 0) sm.par[kRoot] = (uint16_t)kRoot;
    }
    __syncthreads();

    // 3. depths by pointer jumping: dep[v] = distance from v to anc[v]
    const uint32_t v0 = tid, v1 = tid + 256;
    sm.anc[v0] = sm.par[v0];
    sm.dep[v0] = 1;
    if (v1 < kNodes) {
        sm.anc[v1] = sm.par[v1];
        sm.dep[v1] = v1 == kRoot ? 0 : 1;
    }
    __syncthreads();
#pragma unroll 1
    for (int round = 0; round < 9; ++round) {
        const uint32_t a0 = sm.anc[v0];
        const uint32_t d0 = sm.dep[a0], aa0 = sm.anc[a0];
        uint32_t a1 = 0, d1 = 0, aa1 = 0;
        if (v1 < kNodes) {
            a1 = sm.anc[v1];
            d1 = sm.dep[a1];
            aa1 = sm.anc[a1];
        }
        __syncthreads();
        sm.dep[v0] = (uint16_t)(sm.dep[v0] + d0);
        sm.anc[v0] = (uint16_t)aa0;
        if (v1 < kNodes) {
            sm.dep[v1] = (uint16_t)(sm.dep[v1] + d1);
            sm.anc[v1] = (uint16_t)aa1;
        }
        __syncthreads();
    }
    // leaf at sorted position tid: its byte's code length
    const uint32_t d = sm.dep[tid];
    const uint32_t byte = sm.sidx[tid];
    sm.len[byte] = (uint8_t)(d < 255 ? d : 255);
    if (d > (uint32_t)EC_MAX_CODE_LEN) sm.bad = 1;
    else atomicAdd(&sm.blc[d], 1u);
    atomicMax(&sm.max_len, d);
    __syncthreads();

    if (sm.bad) {
        unusable_table(t, tid, status ? status + seg : nullptr, EC_S_BAD_CODEBOOK);
        return;
    }
    canonical_tables(sm, t, tid);
}

// The receiving side of the three-stage design: the tables of the codebook
// a stream carries (its 256 embedded code lengths), so that the decoder
// needs nothing from the encoder but the stream.  A header that is not a
// Huffman stream with embedded lengths, or an index that does not fit in
// in_len, sets EC_S_BAD_HEADER; lengths that are not a complete code of
// 1..EC_MAX_CODE_LEN-bit codes set EC_S_BAD_CODEBOOK.  Either way the table
// is unusable.
__global__ __launch_bounds__(kBuildThreads) void huff_tables_from_streams_kernel(const uint8_t *in,
                                                                                 uint64_t in_stride,
                                                                                 uint64_t in_len, DevTables *tabs,
                                                                                 uint32_t *status) {
    __shared__ BuildSmem sm;
    const uint32_t tid = threadIdx.x;
    const uint32_t seg = blockIdx.x;
    DevTables *t = tabs + seg;
    uint32_t *st = status ? status + seg : nullptr;
    const uint8_t *stream = in + (uint64_t)seg * in_stride;

    const uint64_t *h = reinterpret_cast<const uint64_t *>(stream);
    const uint64_t h0 = h[0], n = h[1], h2 = h[2];
    const uint32_t C = (uint32_t)h2, nch = (uint32_t)(h2 >> 32);
    bool ok = (uint32_t)h0 == kMagic && ((h0 >> 32) & 0xffffu) == kVersion &&
              ((h0 >> 48) & 0xffu) == (uint64_t)EC_CODEC_HUFFMAN && (h0 >> 56) == 1u && n <= (1ull << 33) &&
              C >= kMinChunk && C <= kMaxChunk && C % kSub == 0 && (uint64_t)nch == (n + C - 1) / C;
    const uint64_t lens_at = kHeaderBytes + 8ull * (nch + 1) + 4ull * nch * (C / kSub);
    ok = ok && lens_at + 256 <= in_len;
    if (!ok) {
        unusable_table(t, tid, st, EC_S_BAD_HEADER);
        return;
    }
    if (tid == 0) {
        sm.bad = 0;
        sm.max_len = 0;
    }
    if (tid < 64) sm.blc[tid] = 0;
    __syncthreads();
    const uint32_t l = stream[lens_at + tid];
    sm.len[tid] = (uint8_t)l;
    if (l == 0 || l > (uint32_t)EC_MAX_CODE_LEN) sm.bad = 1;
    else atomicAdd(&sm.blc[l], 1u);
    atomicMax(&sm.max_len, l);
    __syncthreads();
    if (tid == 0) {
        // Kraft sum exactly 1: sum over lengths of count << (40 - length) == 2^40
        uint64_t kraft = 0;
        for (uint32_t j = 1; j <= (uint32_t)EC_MAX_CODE_LEN; ++j)
            kraft += (uint64_t)sm.blc[j] << (EC_MAX_CODE_LEN - j);
        if (kraft != (1ull << EC_MAX_CODE_LEN)) sm.bad = 1;
    }
    __syncthreads();
    if (sm.bad) {
        unusable_table(t, tid, st, EC_S_BAD_CODEBOOK);
        return;
    }
    canonical_tables(sm, t, tid);
}

}  // namespace

hipError_t launch_huff_tables_from_streams(const uint8_t *in, uint64_t in_stride, uint64_t in_len,
                                           uint32_t n_seg, DevTables *tabs, uint32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(huff_tables_from_streams_kernel, dim3(n_seg), dim3(kBuildThreads), 0, s, in, in_stride,
                       in_len, tabs, status);
    return hipGetLastError();
}

hipError_t launch_huff_build(const uint64_t *counts, uint32_t n_seg, DevTables *tabs, uint32_t *status,
                             hipStream_t s) {
    hipLaunchKernelGGL(huff_build_kernel, dim3(n_seg), dim3(kBuildThreads), 0, s, counts, tabs, status);
    return hipGetLastError();
}

}  // namespace ec
