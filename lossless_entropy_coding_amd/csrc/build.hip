// Per-shard Huffman codebooks built on the GPU: the codebook-generation stage
// of the three-stage design ("Single-Stage Huffman Encoder for ML
// Compression", abstract: frequency analysis, codebook generation and
// transmission, encoding), so that a batch of shards goes from histogram rows
// to encoded streams without a trip through host memory.
//
// One workgroup of 1024 threads builds the tables of one shard, bit for bit
// the tables the host builder makes from the same counts:
//   1. weights counts[b] + 1; the leaves in stable order of weight: the rank
//      of the distinct key weight << 8 | b among all 256 (four threads per
//      key, each counting over a quarter of the keys);
//   2. the two-queue merge (leaves in sorted order, merged nodes in creation
//      order; the lighter front is taken, the leaf on a tie), run by one wave.
//      Every step takes the two lightest fronts, so the takes come out as the
//      stable merge of the leaves and the merged nodes, and step k's two
//      takes are the children of merged node k.  The merge records only
//      whether each take was a leaf (a bit a take) and each node's weight.
//      Up to 32 steps at a time: the 64 lightest of the nodes known so far
//      (leaves and merged nodes already made) in merge order, one per lane
//      (a bitonic merge across the lanes), give the next steps' weights as
//      sums of pairs, valid up to the first take the newly made node would
//      displace; when that leaves fewer than four steps, 16 steps follow one
//      at a time in scalar registers;
//   3. from those take bits, every node's parent (take p has parent p / 2),
//      then every merged node's depth by pointer jumping (eight rounds cover
//      the deepest possible tree of 256 leaves), and each leaf's code length;
//   4. canonical codes: the number of codes of each length, the first code
//      and first canonical position of each length, each byte's position in
//      (length, byte) order (the rank of length << 8 | byte);
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

constexpr int kBuildThreads = 1024;
constexpr uint32_t kRootNode = 254;              // merged nodes 0..254; the last one is the root
constexpr uint32_t kTakes = 510;                 // two takes per merge step
constexpr uint32_t kHeavy32 = 0xffffffffu;       // weight of an empty queue front
constexpr uint64_t kHeavy = ~0ull;
constexpr uint64_t kMaxCount = 1ull << 55;       // larger counts could overflow the 64-bit node weights
// Counts below 2^22 keep every node weight (at most 256 * 2^22) within 2^30,
// so that the merge's keys weight << 1 | type fit 32 bits below the heavy
// key, and the sort key weight << 8 | byte in 32 bits.
constexpr uint64_t kNarrowCount = 1ull << 22;

constexpr uint32_t kWin = 64;                    // nodes of each queue a batch of steps looks at

struct BuildSmem {
    uint64_t sw[256 + 2];              // wide weights: leaves in sorted order (+2 heavy)
    uint64_t iw[256 + 2];              // wide weights: merged nodes in creation order (heavy until made)
    alignas(16) uint64_t key64[256];   // wide sort keys
    uint64_t fcode[48];                // first canonical code of each length
    uint32_t sw32[256 + kWin];         // the same as 32-bit weights (heavy past the leaves)
    uint32_t iw32[256 + kWin];
    alignas(16) uint32_t key[256];     // 32-bit sort keys
    uint32_t part[4][256];             // partial ranks
    uint32_t tb[18];                   // take bits: bit p set = the merge's p-th take is a leaf
    uint32_t fidx[48];                 // first canonical position of each length
    alignas(16) uint32_t blc[64];      // codes of each length
    uint32_t lim13[16];                // end of the codes of length l as 13-bit windows
    uint8_t npar[256];                 // parent of merged node j (the root: itself)
    uint8_t lpar[256];                 // parent of the leaf at sorted position i
    uint8_t anc[256];                  // pointer-jumping ancestor of merged node j
    uint8_t dep[256];                  // distance from j to anc[j]
    uint8_t sidx[256];                 // byte at sorted position
    alignas(16) uint8_t len[256];      // code length by byte
    uint8_t symc[256];                 // byte at canonical position
    uint32_t bad, max_len, wide;
};

__device__ __forceinline__ uint32_t rfl(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// FNV-1a 64 (h = (h ^ byte) * P, P = 2^40 + 0x1b3) split in 32-bit halves:
// with y = lo ^ byte, the step is lo' = y * c and hi' = hi * c + g(y), where
// c = 0x1b3 and g(y) = (the high word of y * c) + (y << 8), all modulo 2^32.
// The low words form the only serial chain; the high word after n steps is
// hi_0 c^n + sum_i g(y_i) c^(n-1-i), a sum that lanes add in parallel.  The
// codebook id hashes the codec byte, then the 256 code lengths: the codec
// byte's step is done here.
constexpr uint32_t kFnvC = 0x1b3u;
constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ull;
constexpr uint32_t pow_c(uint32_t e) {
    uint32_t r = 1;
    for (uint32_t i = 0; i < e; ++i) r *= kFnvC;
    return r;
}
constexpr uint32_t fnv_g(uint32_t y) { return (uint32_t)(((uint64_t)y * kFnvC) >> 32) + (y << 8); }
constexpr uint32_t kFnvY0 = (uint32_t)kFnvBasis ^ (uint32_t)EC_CODEC_HUFFMAN;
constexpr uint32_t kFnvLo1 = kFnvY0 * kFnvC;   // low word after the codec byte
// the high word's part from the basis and the codec byte, after all 257 steps
constexpr uint32_t kFnvHiK = (uint32_t)(kFnvBasis >> 32) * pow_c(257) + fnv_g(kFnvY0) * pow_c(256);

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    return (uint64_t)rfl((uint32_t)(x >> 32)) << 32 | rfl((uint32_t)x);
}

// Rank of key[s] among 256 distinct keys (the number of smaller ones) for
// s = tid & 255: thread tid counts over the quarter tid >> 8 of the keys
// (the 64 lanes of a wave read the same key at a time), and thread s adds
// the four partial counts.  Called by every thread after the keys are
// written and a barrier; valid for tid < 256.
template <typename K>
__device__ uint32_t rank_keys(const K *key, uint32_t (*part)[256], uint32_t tid) {
    const uint32_t s = tid & 255u, q = tid >> 8;
    const K ks = key[s];
    const K *kq = key + 64 * q;
    uint32_t r = 0;
#pragma unroll 16
    for (uint32_t j = 0; j < 64; ++j) r += kq[j] < ks ? 1u : 0u;
    part[q][s] = r;
    __syncthreads();
    return tid < 256 ? part[0][s] + part[1][s] + part[2][s] + part[3][s] : 0u;
}

// An unusable table (codec 0, every entry zero), and the status bits saying why.
__device__ void unusable_table(DevTables *t, uint32_t tid, uint32_t *status, uint32_t bits) {
    uint4 *p = reinterpret_cast<uint4 *>(t);
    for (uint32_t i = tid; i < sizeof(DevTables) / 16; i += kBuildThreads) p[i] = make_uint4(0, 0, 0, 0);
    if (tid == 0) or_status(status, bits);
}

// Steps 4 and 5, from the code lengths in sm.len (a complete code, every
// length 1..EC_MAX_CODE_LEN) and their counts sm.blc.  Called by every
// thread of the workgroup.
__device__ void canonical_tables(BuildSmem &sm, DevTables *t, uint32_t tid) {
    const uint32_t wave = tid >> 6;
    if (wave == 0) {
        // the longest length with a code
        const uint64_t used = __ballot(tid < 48 && sm.blc[tid] != 0);
        if (tid == 0) sm.max_len = 63u - (uint32_t)__builtin_clzll(used);
    }
    // 4. canonical codes.  first_code[l] = sum_{j<l} blc[j] << (l - j) and
    // first_idx[l] = sum_{j<l} blc[j] (the recurrence c_l = (c_{l-1} +
    // blc[l-1]) << 1 unrolled).
    // As sum_{j<l} blc[j] << (40 - j), shifted down by 40 - l (every term
    // is a multiple of 2^(40 - l)); the counts are read by all lanes at once.
    if (wave == 0) {
        uint64_t F = 0;
        uint32_t fi = 0;
        const uint4 *bv = reinterpret_cast<const uint4 *>(sm.blc);
#pragma unroll
        for (uint32_t q = 0; q < 11; ++q) {
            const uint4 v = bv[q];
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (uint32_t r = 0; r < 4; ++r) {
                const uint32_t j = 4 * q + r;
                if (j >= 1 && j <= (uint32_t)EC_MAX_CODE_LEN) {
                    const bool in = j < tid;
                    F += in ? (uint64_t)vv[r] << (EC_MAX_CODE_LEN - j) : 0ull;
                    fi += in ? vv[r] : 0u;
                }
            }
        }
        if (tid < 48) {
            const bool in = tid >= 1 && tid <= (uint32_t)EC_MAX_CODE_LEN;
            sm.fcode[tid] = in ? F >> (EC_MAX_CODE_LEN - tid) : 0ull;
            sm.fidx[tid] = in ? fi : 0u;
        }
    }
    // (length, byte) keys for the canonical order
    if (tid < 256) sm.key[tid] = (uint32_t)sm.len[tid] << 8 | tid;
    __syncthreads();
    if (tid >= 1 && tid <= (uint32_t)kHuffBits)
        sm.lim13[tid] = (uint32_t)((sm.fcode[tid] + sm.blc[tid]) << (kHuffBits - tid));
    const uint32_t pos = rank_keys(sm.key, sm.part, tid);
    const uint32_t my_len = tid < 256 ? sm.len[tid] : 0u;
    uint64_t code = 0;
    if (tid < 256) {
        sm.symc[pos] = (uint8_t)tid;
        code = sm.fcode[my_len] + (pos - sm.fidx[my_len]);
    }
    const uint32_t max_len = sm.max_len;
    __syncthreads();

    // 5. tables
    if (tid < 256) {
        t->enc64[tid] = (code << (64 - my_len)) | my_len;
        t->enc32[tid] = max_len <= (uint32_t)kNarrowMaxLen ? ((uint32_t)code << (32 - my_len)) | my_len : 0u;
        t->sym[tid] = sm.symc[tid];
        t->code_len[tid] = (uint8_t)my_len;
    }
    for (uint32_t i = tid; i < (uint32_t)kL1Size * 2 / 16; i += kBuildThreads)
        reinterpret_cast<uint4 *>(t->l1)[i] = make_uint4(0, 0, 0, 0);
    if (tid < 48) {
        const bool in = tid >= 1 && tid <= (uint32_t)EC_MAX_CODE_LEN;
        t->limit[tid] = in ? (sm.fcode[tid] + sm.blc[tid]) << (EC_MAX_CODE_LEN - tid) : 0ull;
        t->first_code[tid] = in ? sm.fcode[tid] : 0ull;
        t->first_idx[tid] = in ? sm.fidx[tid] : 0u;
    }
    if (wave == 0) {
        // codebook id: FNV-1a 64 over the codec byte and the 256 code
        // lengths.  Lane L holds lengths 4 L .. 4 L + 3 (one LDS word).  The
        // low words' chain runs on uniform values in scalar registers, the
        // words brought over by lane reads; lane L keeps the low word before
        // its first length, and redoes its four steps to get their y.
        const uint32_t lane = tid;
        const uint32_t w4 = reinterpret_cast<const uint32_t *>(sm.len)[lane];
        uint32_t lo = kFnvLo1, lo_at = 0;
#pragma unroll 4
        for (uint32_t q = 0; q < 64; ++q) {
            const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)w4, (int)q);
            lo_at = lane == q ? lo : lo_at;
            lo = (lo ^ (w & 0xffu)) * kFnvC;
            lo = (lo ^ ((w >> 8) & 0xffu)) * kFnvC;
            lo = (lo ^ ((w >> 16) & 0xffu)) * kFnvC;
            lo = (lo ^ (w >> 24)) * kFnvC;
        }
        const uint32_t y0 = lo_at ^ (w4 & 0xffu);
        const uint32_t y1 = (y0 * kFnvC) ^ ((w4 >> 8) & 0xffu);
        const uint32_t y2 = (y1 * kFnvC) ^ ((w4 >> 16) & 0xffu);
        const uint32_t y3 = (y2 * kFnvC) ^ (w4 >> 24);
        // lane L's steps (lengths 4 L + r) are followed by 255 - 4 L - r more
        const uint32_t e = 252u - 4u * lane;
        uint32_t base = 1, sq = kFnvC;
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            base = ((e >> bit) & 1u) ? base * sq : base;
            sq *= sq;
        }
        uint32_t part = fnv_g(y3) * base + fnv_g(y2) * (base * kFnvC) + fnv_g(y1) * (base * pow_c(2)) +
                        fnv_g(y0) * (base * pow_c(3));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) part += (uint32_t)__shfl_xor((int)part, o, 64);
        const uint64_t h = (uint64_t)(kFnvHiK + part) << 32 | lo;
        if (tid == 0) {
            t->codebook_id = h;
            t->codec = EC_CODEC_HUFFMAN;
            t->max_len = max_len;
            t->qlc_lens = 0;
            t->eg_k = -1;
            t->pad[0] = 0;
            t->pad[1] = 0;
        }
    } else {
        // 13-bit decode table, eight entries a thread: window w starts a
        // code of length l = 1 + #{l' <= 13 : lim13[l'] <= w}; none when
        // l > 13
        uint32_t lim[kHuffBits + 1];
#pragma unroll
        for (int l = 1; l <= kHuffBits; ++l) lim[l] = sm.lim13[l];
        for (uint32_t u = tid - 64; u < (uint32_t)kHuffSize / 8; u += kBuildThreads - 64) {
            uint32_t e[8];
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) {
                const uint32_t w = 8 * u + k;
                uint32_t l = 1;
#pragma unroll
                for (int j = 1; j <= kHuffBits; ++j) l += lim[j] <= w ? 1u : 0u;
                e[k] = 0;
                if (l <= (uint32_t)kHuffBits) {
                    const uint32_t idx = sm.fidx[l] + ((w >> (kHuffBits - l)) - (uint32_t)sm.fcode[l]);
                    e[k] = l | (uint32_t)sm.symc[idx & 255u] << 8;
                }
            }
            reinterpret_cast<uint4 *>(t->hl1)[u] =
                make_uint4(e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16);
        }
    }
}

// OR a run of take bits (bit i for take pos + i, pos even) into sm.tb.
__device__ __forceinline__ void put_takes(BuildSmem &sm, uint32_t lane, uint32_t pos, uint64_t bits) {
    const uint32_t w = pos >> 5, off = pos & 31u;
    const uint64_t lo = bits << off;
    const uint32_t carry = off ? (uint32_t)(bits >> (64 - off)) : 0u;
    if (lane == 0) {
        sm.tb[w] |= (uint32_t)lo;
        sm.tb[w + 1] |= (uint32_t)(lo >> 32);
        sm.tb[w + 2] |= carry;
    }
}

// Step 2 for weights within 2^30, one wave.  Merged nodes not made yet read
// as heavy (the node array is filled with heavy weights first), and so do
// leaves past the last.
//
// A batch at merge step k (li leaves and qh nodes taken so far): lane p
// gets the item at position p of the stable merge of the next 64 leaves and
// the next 64 nodes, so lanes 2j and 2j + 1 hold the two takes of step
// k + j, if no node made from step k on is taken before them.  Node k, of weight s0 = the sum of
// the first two takes, comes after every known node and leaf no heavier
// than s0 (leaves first on a tie, older nodes first), and the nodes after
// it are heavier still: so the first cnt takes, those no heavier than s0,
// are exact, and cnt / 2 >= 1 steps hold.
//
// The one-at-a-time steps keep every value they depend on in scalar
// registers: the fronts of both queues (L0 L1, Q0 Q1) and the entries that
// may become fronts next (leaves li + 2, li + 3; nodes qh + 2, qh + 3), read
// at the start of each step and taken up at its end; node qt, made in the
// same step, is taken from the step itself.  No branch on the weights, only
// selects.
__device__ void merge32(BuildSmem &sm, uint32_t lane) {
    uint32_t k = 0, li = 0, qh = 0;
    const uint32_t *a = sm.sw32, *b = sm.iw32;
#pragma unroll 1
    while (k < kRootNode + 1) {
        // The 64 lightest of the next 64 leaves and the next 64 nodes, in
        // merge order: keys weight << 1 | (1 for a node), so that a leaf
        // comes first on a tie.  Lane p holds leaf li + p and node qh + 63 -
        // p; the lighter of the two is a bitonic sequence of the 64 lightest,
        // sorted by exchanges with lanes p ^ 32 .. p ^ 1 (swaps of equal keys
        // change nothing that is kept).
        const uint32_t ka = a[li + lane] << 1, kb = b[qh + 63 - lane] << 1 | 1u;
        uint32_t key = ka < kb ? ka : kb;
        auto exchange = [&](uint32_t other, uint32_t d) __attribute__((always_inline)) {
            const uint32_t lo = key < other ? key : other, hi = key < other ? other : key;
            key = (lane & d) ? hi : lo;
        };
        exchange((uint32_t)__shfl_xor((int)key, 32, 64), 32);
        exchange((uint32_t)__builtin_amdgcn_ds_swizzle((int)key, 0x1f | 16 << 10), 16);   // lane ^ 16
        exchange((uint32_t)__builtin_amdgcn_ds_swizzle((int)key, 0x1f | 8 << 10), 8);
        exchange((uint32_t)__builtin_amdgcn_ds_swizzle((int)key, 0x1f | 4 << 10), 4);
        exchange((uint32_t)__builtin_amdgcn_mov_dpp((int)key, 0x4e, 0xf, 0xf, false), 2);   // quad [2 3 0 1]
        exchange((uint32_t)__builtin_amdgcn_mov_dpp((int)key, 0xb1, 0xf, 0xf, false), 1);   // quad [1 0 3 2]
        const bool leaf = (key & 1u) == 0;
        const uint32_t tw = key >> 1;   // heavy entries: above any weight
        // lane 2 j: the weight of node k + j
        const uint32_t pair = (uint32_t)__builtin_amdgcn_mov_dpp((int)tw, 0xb1, 0xf, 0xf, false);   // lane ^ 1
        const uint32_t sum = tw + pair;
        const uint32_t s0 = rfl(sum);
        const uint32_t cnt = (uint32_t)__builtin_popcountll(__ballot(tw <= s0));
        uint32_t m = cnt >> 1;
        if (m > kRootNode + 1 - k) m = kRootNode + 1 - k;
        if (m == 0) m = 1;   // (cnt >= 2: the first two takes are below their sum)
        if ((lane & 1) == 0 && (lane >> 1) < m) sm.iw32[k + (lane >> 1)] = sum;
        const uint64_t taken = 2 * m == 64 ? ~0ull : (1ull << (2 * m)) - 1;
        const uint64_t leaves = __ballot(leaf) & taken;
        put_takes(sm, lane, 2 * k, leaves);
        const uint32_t nl = (uint32_t)__builtin_popcountll(leaves);
        li += nl;
        qh += 2 * m - nl;
        k += m;
        // (the windows stay inside the arrays whatever the weights)
        li = li < 256 ? li : 256u;
        qh = qh < kRootNode ? qh : kRootNode;
        if (m >= 4 || k > kRootNode) continue;

        // a few steps one at a time
        uint32_t steps = kRootNode + 1 - k;
        if (steps > 16) steps = 16;
        uint32_t L0 = rfl(a[li]), L1 = rfl(a[li + 1]), Q0 = rfl(b[qh]), Q1 = rfl(b[qh + 1]);
        uint64_t bits = 0;
#pragma unroll 1
        for (uint32_t j = 0; j < steps; ++j) {
            const uint32_t qt = k + j;
            const uint32_t l2 = a[li + 2], l3 = a[li + 3];
            const uint32_t q2 = b[qh + 2], q3 = b[qh + 3];
            // the first take: the leaf on a tie; the second from what is left
            const bool c0 = L0 <= Q0;
            const uint32_t A = c0 ? L1 : L0, B = c0 ? Q0 : Q1;
            const bool c1 = A <= B;
            const uint32_t s = (c0 ? L0 : Q0) + (c1 ? A : B);
            const uint32_t f = (c0 ? 1u : 0u) | (c1 ? 2u : 0u);
            bits |= (uint64_t)f << (2 * j);
            const uint32_t n = (uint32_t)__builtin_popcount(f);   // leaves taken
            sm.iw32[qt] = s;   // every lane writes the same value
            const uint32_t L2 = rfl(l2), L3 = rfl(l3), Q2 = rfl(q2), Q3 = rfl(q3);
            const bool n0 = n == 0, lt2 = n < 2;
            const uint32_t t0 = n0 ? L0 : L1, t1 = n0 ? L1 : L2;
            const uint32_t u0 = n0 ? Q2 : Q1, u1 = n0 ? Q3 : Q2;
            L0 = lt2 ? t0 : L2;
            L1 = lt2 ? t1 : L3;
            const uint32_t w0 = lt2 ? u0 : Q0, w1 = lt2 ? u1 : Q1;
            const uint32_t qh2 = qh + 2 - n;
            Q0 = qh2 == qt ? s : w0;
            Q1 = qh2 + 1 == qt ? s : w1;
            li += n;
            qh = qh2;
        }
        put_takes(sm, lane, 2 * k, bits);
        k += steps;
    }
}

// Step 2 for wider weights (64-bit; rare), one wave, a step at a time.
__device__ void merge64(BuildSmem &sm) {
    uint32_t li = 0, qh = 0, bits = 0;
#pragma unroll 1
    for (uint32_t k = 0; k <= kRootNode; ++k) {
        const uint64_t L0 = uniform64(sm.sw[li]), L1 = uniform64(sm.sw[li + 1]);
        const uint64_t Q0 = uniform64(sm.iw[qh]), Q1 = uniform64(sm.iw[qh + 1]);
        const bool c0 = L0 <= Q0;
        const uint64_t A = c0 ? L1 : L0, B = c0 ? Q0 : Q1;
        const bool c1 = A <= B;
        const uint64_t sum = (c0 ? L0 : Q0) + (c1 ? A : B);
        const uint32_t f = (c0 ? 1u : 0u) | (c1 ? 2u : 0u);
        bits |= f << (2 * (k & 15));
        if ((k & 15) == 15 || k == kRootNode) {
            sm.tb[k >> 4] = bits;
            bits = 0;
        }
        sm.iw[k] = sum;
        const uint32_t nl = (uint32_t)__builtin_popcount(f);
        li += nl;
        qh += 2 - nl;
    }
}

// Step 3, one wave: parents from the take bits, merged-node depths by
// pointer jumping, the leaves' code lengths and their counts.
__device__ void code_lengths(BuildSmem &sm, uint32_t lane) {
    // lane l: takes p = 8 l .. 8 l + 7.  A take's index among the leaves
    // (merged nodes) is the number of leaves (nodes) taken before it.
    const uint32_t word = sm.tb[lane >> 2], sh = 8 * (lane & 3);
    uint32_t before = (uint32_t)__builtin_popcount(word & ((1u << sh) - 1u));
#pragma unroll
    for (uint32_t i = 0; i < 15; ++i) before += i < (lane >> 2) ? (uint32_t)__builtin_popcount(sm.tb[i]) : 0u;
#pragma unroll
    for (uint32_t b = 0; b < 8; ++b) {
        const uint32_t p = 8 * lane + b;
        const bool leaf = (word >> (sh + b)) & 1u;
        if (p < kTakes) {
            if (leaf) sm.lpar[before] = (uint8_t)(p >> 1);
            else sm.npar[p - before] = (uint8_t)(p >> 1);
        }
        before += leaf ? 1u : 0u;
    }
    // merged nodes v = lane + 64 i keep their ancestor and distance in
    // registers; the root (and the unused slot 255) points at itself
    uint32_t A[4], D[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t v = lane + 64 * i;
        A[i] = v < kRootNode ? sm.npar[v] : kRootNode;
        D[i] = v < kRootNode ? 1u : 0u;
        sm.anc[v] = (uint8_t)A[i];
        sm.dep[v] = (uint8_t)D[i];
    }
    // A wave's LDS operations complete in order: each round's reads see the
    // previous round's writes and none of its own.
#pragma unroll 1
    for (uint32_t round = 0; round < 8; ++round) {
        uint32_t d[4], a[4];
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
            d[i] = sm.dep[A[i]];
            a[i] = sm.anc[A[i]];
        }
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
            const uint32_t v = lane + 64 * i;
            D[i] += d[i];
            A[i] = a[i];
            sm.dep[v] = (uint8_t)D[i];
            sm.anc[v] = (uint8_t)A[i];
        }
    }
    // leaf at sorted position s: one below its parent
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t s = lane + 64 * i;
        const uint32_t d = 1u + sm.dep[sm.lpar[s]];
        sm.len[sm.sidx[s]] = (uint8_t)(d < 255 ? d : 255);
        if (d > (uint32_t)EC_MAX_CODE_LEN) sm.bad = 1;
        else atomicAdd(&sm.blc[d], 1u);
    }
}

__global__ __launch_bounds__(kBuildThreads) void huff_build_kernel(const uint64_t *counts, DevTables *tabs,
                                                                   uint32_t *status) {
    __shared__ BuildSmem sm;
    const uint32_t tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint32_t seg = blockIdx.x;
    DevTables *t = tabs + seg;

    // 1. weights and the stable sort of the leaves
    const uint64_t c = tid < 256 ? counts[(uint64_t)seg * 256 + tid] : 0ull;
    const uint64_t ws = c + 1;
    if (tid == 0) {
        sm.bad = 0;
        sm.max_len = 0;
        sm.wide = 0;
    }
    if (tid < 64) sm.blc[tid] = 0;
    // heavy sentinels past the leaves, and merged nodes not made yet
    if (tid < 256 + kWin) sm.iw32[tid] = kHeavy32;
    if (tid >= 256 && tid < 256 + kWin) sm.sw32[tid] = kHeavy32;
    if (tid < 18) sm.tb[tid] = 0;
    if (tid < 258) sm.iw[tid] = kHeavy;
    if (tid >= 256 && tid < 258) sm.sw[tid] = kHeavy;
    __syncthreads();
    if (tid < 256 && c >= kMaxCount) sm.bad = 1;
    if (tid < 256 && c >= kNarrowCount) sm.wide = 1;
    __syncthreads();   // sm.bad and sm.wide settled
    if (sm.bad) {      // uniform
        unusable_table(t, tid, status ? status + seg : nullptr, EC_S_BAD_CODEBOOK);
        return;
    }
    const bool wide = sm.wide;
    uint32_t r;
    if (!wide) {
        if (tid < 256) sm.key[tid] = (uint32_t)ws << 8 | tid;
        __syncthreads();
        r = rank_keys(sm.key, sm.part, tid);
    } else {
        if (tid < 256) sm.key64[tid] = ws << 8 | tid;
        __syncthreads();
        r = rank_keys(sm.key64, sm.part, tid);
    }
    if (tid < 256) {
        sm.sw[r] = ws;
        sm.sw32[r] = (uint32_t)ws;
        sm.sidx[r] = (uint8_t)tid;
    }
    __syncthreads();

    // 2, 3: one wave
    if (wave == 0) {
        if (!wide) merge32(sm, lane);
        else merge64(sm);
        code_lengths(sm, lane);
    }
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
    if (tid < 256) {
        const uint32_t l = stream[lens_at + tid];
        sm.len[tid] = (uint8_t)l;
        if (l == 0 || l > (uint32_t)EC_MAX_CODE_LEN) sm.bad = 1;
        else atomicAdd(&sm.blc[l], 1u);
    }
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
