// Chunk-parallel decoder.
//
// Every 256-symbol sub-chunk starts at a bit offset recorded in the stream
// index, so one lane decodes one sub-chunk serially and a wave64 decodes 64
// of them side by side.  Each lane streams its bits through a 64-bit
// MSB-aligned buffer refilled 32 bits at a time from a two-word prefetch
// queue (loads are clamped to the payload, so a corrupt index can never make
// a lane read outside the stream).
//   QLC      the 3-bit prefix gives the code length through a packed
//            constant (no memory access on the dependency chain); the top 11
//            bits index a 2048-entry LDS table that yields the byte or flags
//            an unused suffix.
//   Huffman  the top 11 bits index an LDS table: codes of up to 11 bits
//            resolve there; longer codes point to a per-prefix second-level
//            LDS table of up to 8 more bits; deeper codes (rare) are found by
//            comparing a 40-bit window against the canonical code limits.
//   EG       count leading zeros z; the code is 2z + k + 1 bits; rank -> byte
//            through a 256-entry LDS table.
// After its last symbol a lane checks that it stopped exactly where the index
// says its sub-chunk ends.
#include "dev_common.h"

namespace ec {

namespace {

constexpr int kThreads = 256;

struct BitReader {
    const uint32_t *base;   // lane's first payload word
    uint32_t last;          // last readable word, relative to base
    uint64_t buf;           // next stream bits, MSB-aligned
    uint32_t nb;            // valid bits in buf
    uint32_t q0, q1;        // the following two words
    uint32_t nxt;           // next word to fetch, relative to base
    uint64_t base0;         // absolute index of the lane's first word

    __device__ __forceinline__ uint32_t word(uint32_t i) const { return base[i < last ? i : last]; }

    __device__ __forceinline__ void init(const uint32_t *payload, uint32_t n_words, uint64_t bitpos) {
        const uint64_t w0 = bitpos >> 5;
        const uint64_t lastw = n_words - 1;
        const uint64_t b = w0 < lastw ? w0 : lastw;
        base = payload + b;
        last = (uint32_t)(lastw - b);
        const uint32_t o = (uint32_t)(bitpos & 31);
        buf = (((uint64_t)word(0) << 32) | word(1)) << o;
        nb = 64 - o;
        q0 = word(2);
        q1 = word(3);
        nxt = 4;
        base0 = w0;
    }

    // keep at least 32 valid bits
    __device__ __forceinline__ void refill() {
        if (nb <= 32) {
            buf |= (uint64_t)q0 << (32 - nb);
            nb += 32;
            q0 = q1;
            q1 = word(nxt);
            ++nxt;
        }
    }
    __device__ __forceinline__ uint32_t top() const { return (uint32_t)(buf >> 32); }
    __device__ __forceinline__ void skip(uint32_t l) {
        buf <<= l;
        nb -= l;
    }
    // skip l > nb bits (only codes longer than 32 bits can need this)
    __device__ void skip_long(uint32_t l) {
        const uint32_t rest = l - nb;
        buf = 0;
        nb = 0;
        refill();
        skip(rest);
    }
    // 64 stream bits from the current position (valid when nb >= 8)
    __device__ __forceinline__ uint64_t window64() const {
        return buf | (nb <= 32 ? (uint64_t)q0 << (32 - nb) : (uint64_t)q0 >> (nb - 32));
    }
    // absolute bit position of the next unread bit
    __device__ __forceinline__ uint64_t pos() const { return (base0 + nxt - 2) * 32 - nb; }
};

// Huffman code longer than the two table levels: canonical limit search on
// a 40-bit left-justified window.  Returns symbol | length << 8.
__device__ __noinline__ uint32_t huff_deep(uint64_t window, const DevTables *tab) {
    const uint64_t w40 = window >> (64 - EC_MAX_CODE_LEN);
    uint32_t l = kL1Bits + 1;
    const uint32_t mx = tab->max_len;
    while (l < mx && w40 >= tab->limit[l]) ++l;
    const uint64_t code = w40 >> (EC_MAX_CODE_LEN - l);
    const uint32_t idx = tab->first_idx[l] + (uint32_t)(code - tab->first_code[l]);
    return tab->sym[idx & 255] | (l << 8);
}

template <int CODEC, int PERIOD>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeArgs a) {
    __shared__ uint4 l1v[kL1Size * 2 / 16];
    __shared__ uint4 l2v[CODEC == EC_CODEC_HUFFMAN ? kL2Size * 2 / 16 : 1];
    __shared__ uint8_t symtab[256];
    __shared__ uint32_t s_ok, s_C, s_nch, s_spc;
    __shared__ uint64_t s_po, s_pb;
    const uint16_t *l1 = reinterpret_cast<const uint16_t *>(l1v);
    const uint16_t *l2 = reinterpret_cast<const uint16_t *>(l2v);

    const uint32_t tid = threadIdx.x;
    const uint32_t seg = blockIdx.y;
    const DevTables *tab = seg_tables<DecodeArgs>(seg);
    const uint8_t *stream = a.in + (uint64_t)seg * a.in_stride;
    uint32_t *status = a.status ? a.status + seg : nullptr;

    if (CODEC != EC_CODEC_EXP_GOLOMB) l1v[tid] = reinterpret_cast<const uint4 *>(tab->l1)[tid];
    if (CODEC == EC_CODEC_HUFFMAN) l2v[tid] = reinterpret_cast<const uint4 *>(tab->l2)[tid];
    if (CODEC == EC_CODEC_EXP_GOLOMB) symtab[tid] = tab->sym[tid];

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
            uint64_t end = kHeaderBytes + 8ull * (nch + 1) + 4ull * nch * (C / kSub) + ((flags & 1) ? 256 : 0);
            end = (end + 255) / 256 * 256;
            if (po != end || pb % 16 || po + pb > a.in_len || (n > 0 && pb == 0)) bits = EC_S_BAD_HEADER;
        }
        s_ok = bits == 0;
        if (bits && blockIdx.x == 0) or_status(status, bits);
        s_C = C;
        s_nch = nch;
        s_spc = C / kSub;
        s_po = po;
        s_pb = pb;
    }
    __syncthreads();
    if (!s_ok) return;

    const uint32_t g = blockIdx.x * kThreads + tid;   // 256-symbol run within the segment
    if (g >= a.blocks_per_seg) return;
    const uint32_t spc = s_spc;
    const uint32_t c = g / spc, j = g - c * spc;
    const uint64_t *chunk_off = reinterpret_cast<const uint64_t *>(stream + kHeaderBytes);
    const uint32_t *sub_end = reinterpret_cast<const uint32_t *>(stream + kHeaderBytes + 8ull * (s_nch + 1));
    const uint64_t co0 = chunk_off[c], co1 = chunk_off[c + 1];
    const uint32_t e_end = sub_end[(uint64_t)c * spc + j];
    const uint32_t e_start = j ? sub_end[(uint64_t)c * spc + j - 1] : 0u;
    if (co0 > co1 || co1 > s_pb || (co0 & 15) || (uint64_t)e_end > (co1 - co0) * 8 || e_start > e_end) {
        or_status(status, EC_S_CORRUPT);
        return;
    }
    const uint64_t first_sym = (uint64_t)g * kSub;
    const uint32_t cnt = a.seg_n - first_sym < kSub ? (uint32_t)(a.seg_n - first_sym) : (uint32_t)kSub;

    BitReader R;
    R.init(reinterpret_cast<const uint32_t *>(stream + s_po), (uint32_t)(s_pb >> 2), co0 * 8 + e_start);

    const uint32_t lens = tab->qlc_lens;
    const uint32_t k_eg = (uint32_t)tab->eg_k;
    uint32_t bad = 0;

    auto step = [&]() -> uint32_t {
        const uint32_t t = R.top();
        if (CODEC == EC_CODEC_QLC) {
            const uint32_t e = l1[t >> 21];
            bad |= e;
            R.skip((lens >> ((t >> 29) << 2)) & 15u);
            return e & 0xffu;
        } else if (CODEC == EC_CODEC_HUFFMAN) {
            uint32_t e = l1[t >> 21];
            if (e & kL1Long) {
                const uint32_t w2 = ((e >> 12) & 7u) + 1u;
                e = l2[(e & 0x7ffu) + ((t << kL1Bits) >> (32u - w2))];
                if ((e >> 8) == 0) e = huff_deep(R.window64(), tab);
            }
            const uint32_t l = e >> 8;
            if (l <= R.nb)
                R.skip(l);
            else
                R.skip_long(l);
            return e & 0xffu;
        } else {
            uint32_t z = __clz(t);
            if (z > 8) {
                bad |= kQlcInvalid;
                z = 8;
            }
            const uint32_t l = 2 * z + k_eg + 1;
            const uint32_t rank = (t >> (32 - l)) - (1u << k_eg);
            if (rank > 255) bad |= kQlcInvalid;
            R.skip(l);
            return symtab[rank & 255u];
        }
    };

    uint8_t *dst = a.out + (uint64_t)seg * a.out_stride + first_sym;
    if (cnt == kSub) {
        for (int i = 0; i < kSub / 16; ++i) {
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (k % PERIOD == 0) R.refill();
                w[k >> 2] |= step() << (8 * (k & 3));
            }
            *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        for (uint32_t k = 0; k < cnt; ++k) {
            R.refill();
            dst[k] = (uint8_t)step();
        }
    }
    if ((bad & kQlcInvalid) || R.pos() != ((uint64_t)co0 * 8 + e_end)) or_status(status, EC_S_CORRUPT);
}

template <int CODEC, int PERIOD>
hipError_t launch_one(const DecodeArgs &a, hipStream_t s) {
    uint32_t gx = (a.blocks_per_seg + kThreads - 1) / kThreads;
    if (gx == 0) gx = 1;   // still validate the header
    hipLaunchKernelGGL((decode_kernel<CODEC, PERIOD>), dim3(gx, a.n_seg), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, uint32_t codec, uint32_t /*max_len*/, hipStream_t s) {
    switch (codec) {
        case EC_CODEC_QLC:
            return launch_one<EC_CODEC_QLC, 2>(a, s);   // codes <= 11 bits: 2 per 32 buffered bits
        case EC_CODEC_HUFFMAN:
            return launch_one<EC_CODEC_HUFFMAN, 1>(a, s);
        default:
            return launch_one<EC_CODEC_EXP_GOLOMB, 1>(a, s);
    }
}

}  // namespace ec
