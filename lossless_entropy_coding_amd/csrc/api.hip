// C ABI of libec: argument checks, per-device state and kernel launches.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "dev_common.h"

// Chunk sizes of entropy_encode_noalloc, in a fixed device array instead of
// allocated scratch: one u32 per chunk, up to 65536 chunks a call.  In host
// code the name `scratch` only stands for the symbol; kernels get the array's
// device address on each device, looked up once per device.
static __device__ __align__(256) uint32_t scratch[65536];

namespace ec {
namespace {

constexpr uint64_t kNoAllocChunks = sizeof(scratch) / sizeof(scratch[0]);

constexpr uint64_t kMaxSegSymbols = 1ull << 33;   // per stream
constexpr int kMaxDevices = 16;

// Scratch of one device and stream, one buffer per use: the encoder's chunk
// sizes, the histogram's partial counts, and the BF16 encoder's per-chunk
// escape counts and staged escapes.  Calls on one stream run in order, so
// they may share; calls on different streams have buffers of their own.
// Grown by doubling; retired buffers are kept (a kernel still in flight may
// use them) until the process ends.
enum ScratchSlot { kScratchSizes = 0, kScratchHist = 1, kScratchBfCounts = 2, kScratchBfEsc = 3, kScratchSlots = 4 };

struct StreamScratch {
    void *buf[kScratchSlots] = {};
    uint64_t bytes[kScratchSlots] = {};
};

struct DeviceState {
    std::mutex mu;
    std::unordered_map<hipStream_t, StreamScratch> by_stream;
    std::vector<void *> retired;
};

DeviceState g_dev[kMaxDevices];

int current_device(int *dev) {
    if (hipGetDevice(dev) != hipSuccess) return EC_E_HIP;
    if (*dev < 0 || *dev >= kMaxDevices) return EC_E_UNSUPPORTED;
    return EC_OK;
}

// At least `bytes` of scratch `slot` for work on `stream` on the current device.
int device_scratch(int slot, uint64_t bytes, hipStream_t stream, void **out) {
    int dev;
    int rc = current_device(&dev);
    if (rc) return rc;
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    StreamScratch &sc = d.by_stream[stream];
    if (bytes > sc.bytes[slot]) {
        uint64_t cap = sc.bytes[slot] ? sc.bytes[slot] : (1u << 18);
        while (cap < bytes) cap *= 2;
        void *p = nullptr;
        if (hipMalloc(&p, cap) != hipSuccess) return EC_E_NOMEM;
        if (sc.buf[slot]) d.retired.push_back(sc.buf[slot]);
        sc.buf[slot] = p;
        sc.bytes[slot] = cap;
    }
    *out = sc.buf[slot];
    return EC_OK;
}

// Device copy of a codebook's tables on the current device.
int device_tables(const ec_codebook *cbc, const DevTables **out) {
    ec_codebook *cb = const_cast<ec_codebook *>(cbc);
    int dev;
    int rc = current_device(&dev);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(cb->mu);
    if (!cb->dev[dev]) {
        DevTables *p = nullptr;
        if (hipMalloc(&p, sizeof(DevTables)) != hipSuccess) return EC_E_NOMEM;
        if (hipMemcpy(p, &cb->host, sizeof(DevTables), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(p);
            return EC_E_HIP;
        }
        cb->dev[dev] = p;
    }
    *out = cb->dev[dev];
    return EC_OK;
}

// The codebook's tables on the current device if an earlier call put them
// there (no allocation): EC_E_INVAL otherwise.
int resident_tables(const ec_codebook *cbc, const DevTables **out) {
    ec_codebook *cb = const_cast<ec_codebook *>(cbc);
    int dev;
    int rc = current_device(&dev);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(cb->mu);
    if (!cb->dev[dev]) return EC_E_INVAL;
    *out = cb->dev[dev];
    return EC_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool chunk_ok(uint32_t C) { return C >= kMinChunk && C <= kMaxChunk && C % kSub == 0; }

struct Layout {
    uint64_t n_chunks, sub_at, index_end, payload_offset;
};

Layout layout(uint64_t n, uint32_t C, uint32_t embed) {
    Layout l;
    l.n_chunks = (n + C - 1) / C;
    l.sub_at = kHeaderBytes + 8 * (l.n_chunks + 1);
    l.index_end = l.sub_at + 4 * l.n_chunks * (C / kSub) + (embed ? 256 : 0);
    l.payload_offset = (l.index_end + 255) / 256 * 256;
    return l;
}

uint64_t max_payload(uint64_t n, uint32_t C, uint32_t max_len) {
    const uint64_t full = n / C, rest = n % C;
    auto chunk_bytes = [&](uint64_t syms) { return ((syms * max_len + 7) / 8 + 15) / 16 * 16; };
    return full * chunk_bytes(C) + (rest ? chunk_bytes(rest) : 0);
}

int hip_rc(hipError_t e) { return e == hipSuccess ? EC_OK : EC_E_HIP; }

// Where a launch's codebook tables come from: library handles (uploaded on
// first use, their sizes known to the host) or a caller-owned device array of
// tables the host never reads.
struct TableSrc {
    const ec_codebook *const *cbs;
    const uint8_t *dev;
};

const DevTables *dev_table(const uint8_t *base, uint32_t i) {
    return reinterpret_cast<const DevTables *>(base + (uint64_t)i * sizeof(DevTables));
}

// fixed_sizes: chunk-size scratch the caller provides (fixed_chunks entries;
// the codebook tables must then already be resident), else library scratch.
// given_sizes: the chunk sizes themselves, made by byte_histogram_sized (no
// sizes launch).
int encode_impl(TableSrc ts, uint32_t n_seg, const uint8_t *d_in, uint64_t seg_n,
                uint64_t in_stride, uint32_t C, uint32_t embed, uint8_t *d_out, uint64_t out_stride,
                uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status, hipStream_t s,
                uint32_t *fixed_sizes = nullptr, uint64_t fixed_chunks = 0,
                const uint32_t *given_sizes = nullptr) {
    if ((!ts.cbs && !ts.dev) || n_seg == 0 || n_seg > EC_MAX_BATCH || !d_out || !d_out_len || !chunk_ok(C))
        return EC_E_INVAL;
    if (seg_n > kMaxSegSymbols || (seg_n && !d_in) || !aligned16(ts.dev)) return EC_E_INVAL;
    if (!aligned16(d_in) || !aligned16(d_out)) return EC_E_INVAL;
    if (n_seg > 1 && (in_stride % 16 || out_stride % 16 || in_stride < seg_n || out_stride < out_cap))
        return EC_E_INVAL;
    const Layout L = layout(seg_n, C, embed);
    if (L.payload_offset >= (1ull << 32) || L.n_chunks * n_seg >= (1ull << 31)) return EC_E_UNSUPPORTED;
    if (out_cap < L.payload_offset) return EC_E_CAPACITY;

    EncodeArgs a;
    memset(&a, 0, sizeof(a));
    uint32_t max_len = 1;
    for (uint32_t i = 0; i < n_seg; ++i) {
        if (ts.dev) {
            a.tabs[i] = dev_table(ts.dev, i);
            continue;
        }
        const ec_codebook *cb = ts.cbs[i];
        if (!cb) return EC_E_INVAL;
        int rc = fixed_sizes ? resident_tables(cb, &a.tabs[i]) : device_tables(cb, &a.tabs[i]);
        if (rc) return rc;
        max_len = cb->host.max_len > max_len ? cb->host.max_len : max_len;
        if (embed && cb->host.codec != EC_CODEC_HUFFMAN) return EC_E_INVAL;
    }
    if (ts.dev) {
        max_len = EC_MAX_CODE_LEN;
        a.tables_unread = 1;
    }
    a.in = d_in;
    a.in_stride = in_stride;
    a.seg_n = seg_n;
    a.out = d_out;
    a.out_stride = out_stride;
    a.out_cap = out_cap;
    a.out_len = d_out_len;
    a.status = d_status;
    a.chunk_symbols = C;
    a.chunks_per_seg = (uint32_t)L.n_chunks;
    a.n_seg = n_seg;
    a.payload_offset = (uint32_t)L.payload_offset;
    a.sub_at = (uint32_t)L.sub_at;
    a.embed_lengths = embed ? 1 : 0;
    a.max_len = max_len;
    if (given_sizes) {
        if (ts.dev) return EC_E_INVAL;
        if (!encode_sized_supported(C, max_len)) return EC_E_UNSUPPORTED;
        if ((uintptr_t)given_sizes & 3) return EC_E_INVAL;
        a.sized = 1;
        a.sizes = const_cast<uint32_t *>(given_sizes);   // only read
    } else if (L.n_chunks && fixed_sizes) {
        if (L.n_chunks * n_seg > fixed_chunks) return EC_E_UNSUPPORTED;
        a.sizes = fixed_sizes;
    } else if (L.n_chunks) {
        void *p = nullptr;
        int rc = device_scratch(kScratchSizes, L.n_chunks * n_seg * 4, s, &p);
        if (rc) return rc;
        a.sizes = static_cast<uint32_t *>(p);
    }
    return hip_rc(launch_encode(a, s));
}

// codec: the tables' codec when they come from device memory (ts.dev).
int decode_impl(TableSrc ts, uint32_t codec, uint32_t n_seg, const uint8_t *d_in, uint64_t in_stride,
                uint64_t in_len, uint8_t *d_out, uint64_t seg_n, uint64_t out_stride, uint32_t *d_status,
                hipStream_t s) {
    if ((!ts.cbs && !ts.dev) || n_seg == 0 || n_seg > EC_MAX_BATCH || !d_in || in_len < kHeaderBytes)
        return EC_E_INVAL;
    if (seg_n > kMaxSegSymbols || (seg_n && !d_out) || !aligned16(ts.dev)) return EC_E_INVAL;
    if (!aligned16(d_in) || !aligned16(d_out)) return EC_E_INVAL;
    if (n_seg > 1 && (in_stride % 16 || out_stride % 16 || in_stride < in_len || out_stride < seg_n))
        return EC_E_INVAL;
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    uint32_t max_len = EC_MAX_CODE_LEN;
    if (ts.dev) {
        if (codec < EC_CODEC_QLC || codec > EC_CODEC_EXP_GOLOMB) return EC_E_INVAL;
        for (uint32_t i = 0; i < n_seg; ++i) a.tabs[i] = dev_table(ts.dev, i);
    } else {
        codec = ts.cbs[0] ? ts.cbs[0]->host.codec : 0;
        max_len = 0;
        for (uint32_t i = 0; i < n_seg; ++i) {
            if (!ts.cbs[i] || ts.cbs[i]->host.codec != codec) return EC_E_INVAL;
            int rc = device_tables(ts.cbs[i], &a.tabs[i]);
            if (rc) return rc;
            max_len = ts.cbs[i]->host.max_len > max_len ? ts.cbs[i]->host.max_len : max_len;
        }
    }
    a.in = d_in;
    a.in_stride = in_stride;
    a.in_len = in_len;
    a.out = d_out;
    a.out_stride = out_stride;
    a.seg_n = seg_n;
    a.status = d_status;
    a.n_seg = n_seg;
    a.blocks_per_seg = (uint32_t)((seg_n + kSub - 1) / kSub);
    return hip_rc(launch_decode(a, codec, max_len, s));
}

struct ScratchAddr {
    std::once_flag once;
    uint32_t *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchAddr g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with it current).
int noalloc_scratch(uint32_t **out) {
    int dev;
    int rc = current_device(&dev);
    if (rc) return rc;
    ScratchAddr &sa = g_scratch_addr[dev];
    std::call_once(sa.once, [&] { sa.err = hipGetSymbolAddress((void **)&sa.ptr, HIP_SYMBOL(scratch)); });
    if (sa.err != hipSuccess || !sa.ptr) return EC_E_HIP;
    *out = sa.ptr;
    return EC_OK;
}

}  // namespace
}  // namespace ec

using namespace ec;

extern "C" {

const char *ec_error_string(int code) {
    switch (code) {
        case EC_OK: return "ok";
        case EC_E_INVAL: return "invalid argument";
        case EC_E_UNSUPPORTED: return "unsupported";
        case EC_E_NOMEM: return "out of memory";
        case EC_E_HIP: return "HIP runtime error";
        case EC_E_CAPACITY: return "output capacity too small for header and index";
        default: return "unknown error";
    }
}

const char *ec_status_string(uint32_t st) {
    if (st == 0) return "ok";
    if (st & EC_S_BAD_CODEBOOK) return "device-built codebook unusable (code longer than EC_MAX_CODE_LEN)";
    if (st & EC_S_BAD_HEADER) return "bad stream header";
    if (st & EC_S_CODEBOOK_MISMATCH) return "stream made with another codebook";
    if (st & EC_S_CORRUPT) return "corrupt stream";
    if (st & EC_S_CAPACITY) return "output capacity exceeded";
    return "unknown status";
}

int qlc_build_codebook(const uint64_t counts[256], const uint16_t area_size[8], const uint8_t suffix_bits[8],
                       ec_codebook **out) {
    return build_qlc(counts, area_size, suffix_bits, out);
}

int qlc_optimal_area_layout(const uint64_t counts[256], uint32_t max_lengths, uint16_t area_size[8],
                            uint8_t suffix_bits[8]) {
    return qlc_optimal_areas(counts, max_lengths, area_size, suffix_bits);
}

int huff_build_codebook(const uint64_t counts[256], ec_codebook **out) {
    if (!counts || !out) return EC_E_INVAL;
    uint64_t w[256];
    for (int s = 0; s < 256; ++s) {
        if (counts[s] >= (1ull << 55)) return EC_E_INVAL;   // node weights must not overflow
        w[s] = counts[s] + 1;
    }
    uint8_t len[256];
    int rc = huffman_lengths(w, 256, len);
    if (rc) return rc;
    return build_huffman_lengths(len, out);
}

int huff_build_codebook_from_lengths(const uint8_t code_len[256], ec_codebook **out) {
    return build_huffman_lengths(code_len, out);
}

int eg_build_codebook(const uint64_t counts[256], int k, ec_codebook **out) { return build_eg(counts, k, out); }

int huff_code_lengths(const uint64_t *weights, uint32_t n, uint8_t *len_out) {
    return huffman_lengths(weights, n, len_out);
}

int ec_codebook_info(const ec_codebook *cb, uint32_t *codec, uint32_t *max_len, uint64_t *codebook_id,
                     uint8_t code_len[256], uint64_t code[256], uint8_t rank_to_sym[256], int32_t *eg_k) {
    if (!cb) return EC_E_INVAL;
    const DevTables &t = cb->host;
    if (codec) *codec = t.codec;
    if (max_len) *max_len = t.max_len;
    if (codebook_id) *codebook_id = t.codebook_id;
    if (code_len) memcpy(code_len, t.code_len, 256);
    if (code)
        for (int s = 0; s < 256; ++s) code[s] = t.code_len[s] ? t.enc64[s] >> (64 - t.code_len[s]) : 0;
    if (rank_to_sym) {
        if (t.codec == EC_CODEC_HUFFMAN)
            memset(rank_to_sym, 0, 256);
        else
            memcpy(rank_to_sym, t.sym, 256);
    }
    if (eg_k) *eg_k = t.eg_k;
    return EC_OK;
}

void ec_codebook_free(ec_codebook *cb) {
    if (!cb) return;
    for (int d = 0; d < kMaxDevices; ++d)
        if (cb->dev[d]) {
            int cur = 0;
            (void)hipGetDevice(&cur);
            (void)hipSetDevice(d);
            (void)hipFree(cb->dev[d]);
            (void)hipSetDevice(cur);
        }
    delete cb;
}

uint64_t entropy_index_bytes(uint64_t n, uint32_t chunk_symbols, uint32_t embed_lengths) {
    if (!chunk_ok(chunk_symbols) || n > kMaxSegSymbols) return 0;
    return layout(n, chunk_symbols, embed_lengths).payload_offset;
}

uint64_t entropy_max_encoded_bytes(const ec_codebook *cb, uint64_t n, uint32_t chunk_symbols,
                                   uint32_t embed_lengths) {
    if (!cb || !chunk_ok(chunk_symbols) || n > kMaxSegSymbols) return 0;
    return layout(n, chunk_symbols, embed_lengths).payload_offset + max_payload(n, chunk_symbols, cb->host.max_len);
}

int entropy_encode(const ec_codebook *cb, const uint8_t *d_in, uint64_t n, uint32_t chunk_symbols, uint8_t *d_out,
                   uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status, hipStream_t stream) {
    const ec_codebook *cbs[1] = {cb};
    return encode_impl(TableSrc{cbs, nullptr}, 1, d_in, n, 0, chunk_symbols, 0, d_out, 0, out_cap, d_out_len,
                       d_status, stream);
}

int entropy_encode_noalloc(const ec_codebook *cb, const uint8_t *d_in, uint64_t n, uint32_t chunk_symbols,
                           uint8_t *d_out, uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status,
                           hipStream_t stream) {
    if (!chunk_ok(chunk_symbols)) return EC_E_INVAL;
    if ((n + chunk_symbols - 1) / chunk_symbols > kNoAllocChunks) return EC_E_UNSUPPORTED;
    uint32_t *sizes = nullptr;
    int rc = noalloc_scratch(&sizes);
    if (rc) return rc;
    const ec_codebook *cbs[1] = {cb};
    return encode_impl(TableSrc{cbs, nullptr}, 1, d_in, n, 0, chunk_symbols, 0, d_out, 0, out_cap, d_out_len,
                       d_status, stream, sizes, kNoAllocChunks);
}

int entropy_encode_sized(const ec_codebook *cb, const uint8_t *d_in, uint64_t n, uint32_t chunk_symbols,
                         const uint32_t *d_sizes, uint8_t *d_out, uint64_t out_cap, uint64_t *d_out_len,
                         uint32_t *d_status, hipStream_t stream) {
    if (!d_sizes && n) return EC_E_INVAL;
    const ec_codebook *cbs[1] = {cb};
    return encode_impl(TableSrc{cbs, nullptr}, 1, d_in, n, 0, chunk_symbols, 0, d_out, 0, out_cap, d_out_len,
                       d_status, stream, nullptr, 0, n ? d_sizes : nullptr);
}

int entropy_encode_batch_sized(const ec_codebook *const *cbs, uint32_t n_seg, const uint8_t *d_in, uint64_t seg_n,
                               uint64_t in_stride, uint32_t chunk_symbols, uint32_t embed_lengths,
                               const uint32_t *d_sizes, uint8_t *d_out, uint64_t out_stride, uint64_t *d_out_len,
                               uint32_t *d_status, hipStream_t stream) {
    if (!cbs || (!d_sizes && seg_n)) return EC_E_INVAL;
    return encode_impl(TableSrc{cbs, nullptr}, n_seg, d_in, seg_n, in_stride, chunk_symbols, embed_lengths, d_out,
                       out_stride, out_stride, d_out_len, d_status, stream, nullptr, 0, seg_n ? d_sizes : nullptr);
}

int entropy_decode(const ec_codebook *cb, const uint8_t *d_in, uint64_t in_len, uint8_t *d_out, uint64_t n,
                   uint32_t *d_status, hipStream_t stream) {
    const ec_codebook *cbs[1] = {cb};
    return decode_impl(TableSrc{cbs, nullptr}, 0, 1, d_in, 0, in_len, d_out, n, 0, d_status, stream);
}

int entropy_encode_batch(const ec_codebook *const *cbs, uint32_t n_seg, const uint8_t *d_in, uint64_t seg_n,
                         uint64_t in_stride, uint32_t chunk_symbols, uint32_t embed_lengths, uint8_t *d_out,
                         uint64_t out_stride, uint64_t *d_out_len, uint32_t *d_status, hipStream_t stream) {
    if (!cbs) return EC_E_INVAL;
    return encode_impl(TableSrc{cbs, nullptr}, n_seg, d_in, seg_n, in_stride, chunk_symbols, embed_lengths, d_out,
                       out_stride, out_stride, d_out_len, d_status, stream);
}

int entropy_decode_batch(const ec_codebook *const *cbs, uint32_t n_seg, const uint8_t *d_in, uint64_t in_stride,
                         uint8_t *d_out, uint64_t seg_n, uint64_t out_stride, uint32_t *d_status,
                         hipStream_t stream) {
    if (!cbs) return EC_E_INVAL;
    return decode_impl(TableSrc{cbs, nullptr}, 0, n_seg, d_in, in_stride, in_stride, d_out, seg_n, out_stride,
                       d_status, stream);
}

uint64_t ec_device_codebook_bytes(void) { return sizeof(DevTables); }

int huff_build_codebooks_device(const uint64_t *d_counts, uint32_t n_seg, void *d_tables, uint32_t *d_status,
                                hipStream_t stream) {
    if (!d_counts || !d_tables || n_seg == 0 || n_seg > 65535 || !aligned16(d_tables)) return EC_E_INVAL;
    return hip_rc(launch_huff_build(d_counts, n_seg, static_cast<DevTables *>(d_tables), d_status, stream));
}

int huff_tables_from_streams_device(const uint8_t *d_in, uint64_t in_stride, uint64_t in_len, uint32_t n_seg,
                                    void *d_tables, uint32_t *d_status, hipStream_t stream) {
    if (!d_in || !d_tables || n_seg == 0 || n_seg > 65535 || in_len < kHeaderBytes) return EC_E_INVAL;
    if (!aligned16(d_in) || !aligned16(d_tables) || (n_seg > 1 && (in_stride % 16 || in_stride < in_len)))
        return EC_E_INVAL;
    return hip_rc(launch_huff_tables_from_streams(d_in, in_stride, in_len, n_seg, static_cast<DevTables *>(d_tables),
                                                  d_status, stream));
}

int ec_codebook_export(const ec_codebook *cb, void *table) {
    if (!cb || !table) return EC_E_INVAL;
    memcpy(table, &cb->host, sizeof(DevTables));
    return EC_OK;
}

uint64_t entropy_own_max_encoded_bytes(uint64_t n, uint32_t chunk_symbols, uint32_t embed_lengths) {
    if (!chunk_ok(chunk_symbols) || n > kMaxSegSymbols) return 0;
    const Layout l = layout(n, chunk_symbols, embed_lengths);
    return l.payload_offset + n + 16 * l.n_chunks;
}

int entropy_encode_batch_device(const void *d_tables, uint32_t n_seg, const uint8_t *d_in, uint64_t seg_n,
                                uint64_t in_stride, uint32_t chunk_symbols, uint32_t embed_lengths,
                                uint8_t *d_out, uint64_t out_stride, uint64_t *d_out_len, uint32_t *d_status,
                                hipStream_t stream) {
    if (!d_tables) return EC_E_INVAL;
    return encode_impl(TableSrc{nullptr, static_cast<const uint8_t *>(d_tables)}, n_seg, d_in, seg_n, in_stride,
                       chunk_symbols, embed_lengths, d_out, out_stride, out_stride, d_out_len, d_status, stream);
}

int entropy_decode_batch_device(const void *d_tables, uint32_t codec, uint32_t n_seg, const uint8_t *d_in,
                                uint64_t in_stride, uint8_t *d_out, uint64_t seg_n, uint64_t out_stride,
                                uint32_t *d_status, hipStream_t stream) {
    if (!d_tables) return EC_E_INVAL;
    return decode_impl(TableSrc{nullptr, static_cast<const uint8_t *>(d_tables)}, codec, n_seg, d_in, in_stride,
                       in_stride, d_out, seg_n, out_stride, d_status, stream);
}

int byte_histogram(const uint8_t *d_in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride, uint64_t *d_counts,
                   hipStream_t stream) {
    if (!d_counts || n_seg == 0 || n_seg > 65535 || (seg_n && !d_in)) return EC_E_INVAL;
    if (n_seg > 1 && in_stride < seg_n) return EC_E_INVAL;
    if (seg_n >= (1ull << 40)) return EC_E_UNSUPPORTED;
    void *partial = nullptr;
    int rc = device_scratch(kScratchHist, (uint64_t)histogram_blocks(seg_n, n_seg) * n_seg * 1024, stream, &partial);
    if (rc) return rc;
    return hip_rc(launch_histogram(d_in, seg_n, n_seg, in_stride, d_counts, static_cast<uint32_t *>(partial),
                                   nullptr, stream));
}

int byte_histogram_sized(const uint8_t *d_in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride, uint64_t *d_counts,
                         const ec_codebook *const *cbs, uint32_t n_cb, uint32_t chunk_symbols, uint32_t *d_sizes,
                         hipStream_t stream) {
    if (!d_counts || n_seg == 0 || n_seg > 65535 || (seg_n && !d_in)) return EC_E_INVAL;
    if (!cbs || n_cb == 0 || n_cb > kMaxSizeCodebooks || !d_sizes || ((uintptr_t)d_sizes & 3)) return EC_E_INVAL;
    if (!chunk_ok(chunk_symbols)) return EC_E_INVAL;
    if (n_seg > 1 && (in_stride < seg_n || in_stride % 16)) return EC_E_INVAL;
    if (!aligned16(d_in)) return EC_E_INVAL;
    if (seg_n > kMaxSegSymbols) return EC_E_UNSUPPORTED;
    if (!histogram_can_size(seg_n, n_seg, chunk_symbols)) return EC_E_UNSUPPORTED;
    ChunkSizeArgs cs;
    memset(&cs, 0, sizeof(cs));
    for (uint32_t i = 0; i < n_cb; ++i) {
        if (!cbs[i]) return EC_E_INVAL;
        int rc = device_tables(cbs[i], &cs.tabs[i]);
        if (rc) return rc;
    }
    cs.sizes = d_sizes;
    cs.n_cb = n_cb;
    cs.vc_log2 = (uint32_t)__builtin_ctz(chunk_symbols / 16);
    cs.chunks_per_seg = (uint32_t)((seg_n + chunk_symbols - 1) / chunk_symbols);
    void *partial = nullptr;
    int rc = device_scratch(kScratchHist, (uint64_t)histogram_blocks(seg_n, n_seg, true) * n_seg * 1024, stream,
                            &partial);
    if (rc) return rc;
    return hip_rc(launch_histogram(d_in, seg_n, n_seg, in_stride, d_counts, static_cast<uint32_t *>(partial), &cs,
                                   stream));
}

int pmf_average(const uint64_t *d_counts, uint32_t n_seg, float *d_pmf, hipStream_t stream) {
    if (!d_pmf || (n_seg && !d_counts)) return EC_E_INVAL;
    return hip_rc(launch_pmf_average(d_counts, n_seg, d_pmf, stream));
}

int pmf_kl(const uint64_t *d_p, uint32_t n_seg, const uint64_t *d_q, uint32_t q_add, float *d_kl_bits,
           hipStream_t stream) {
    if (!d_q || !d_kl_bits || (n_seg && !d_p) || n_seg > (1u << 30)) return EC_E_INVAL;
    return hip_rc(launch_pmf_kl(d_p, n_seg, d_q, q_add, d_kl_bits, stream));
}

}  // extern "C"

// ------------------------------------------------------------ BF16 exponents

namespace ec {
namespace {

constexpr uint32_t kBfRow = 2048;          // values per row of the kernels
constexpr uint32_t kBfMaxChunks = 8192;    // chunks per stream (the placement sums them per workgroup)

struct BfLayout {
    uint64_t n_chunks, sm_at, plane_at, plane_bytes, esc_at;
};

BfLayout bf_layout(uint64_t n, uint32_t chunk) {
    BfLayout l;
    l.n_chunks = (n + chunk - 1) / chunk;
    const uint64_t idx_end = kHeaderBytes + 8 * (l.n_chunks + 1);
    l.sm_at = (idx_end + 255) / 256 * 256;
    l.plane_at = (l.sm_at + n + 15) / 16 * 16;
    l.plane_bytes = ((n + 7) / 8 + 15) / 16 * 16;
    l.esc_at = l.plane_at + 3 * l.plane_bytes;
    return l;
}

bool bf_chunk_ok(uint32_t chunk) { return chunk >= kBfRow && chunk <= (1u << 20) && chunk % kBfRow == 0; }

}  // namespace
}  // namespace ec

using namespace ec;

int bf16_exp_table_from_counts(const uint64_t counts[256], uint8_t table[7]) {
    if (!counts || !table) return EC_E_INVAL;
    int order[256];
    for (int e = 0; e < 256; ++e) order[e] = e;
    std::stable_sort(order, order + 256, [&](int x, int y) { return counts[x] > counts[y]; });
    for (int k = 0; k < 7; ++k) table[k] = (uint8_t)order[k];
    return EC_OK;
}

int bf16_exp_table_from_sigma(double sigma, uint8_t table[7]) {
    if (!table || !(sigma > 0) || !std::isfinite(sigma)) return EC_E_INVAL;
    // Gaussian mass of the octave of exponent e: |x| in [2^(e-127), 2^(e-126)),
    // [0, 2^-126) for e = 0
    double mass[255];
    const double s = sigma * std::sqrt(2.0);
    for (int e = 0; e < 255; ++e) {
        const double lo = e == 0 ? 0.0 : std::ldexp(1.0, e - 127), hi = std::ldexp(1.0, e - 126);
        mass[e] = std::erf(hi / s) - std::erf(lo / s);
    }
    int order[255];
    for (int e = 0; e < 255; ++e) order[e] = e;
    std::stable_sort(order, order + 255, [&](int x, int y) { return mass[x] > mass[y]; });
    for (int k = 0; k < 7; ++k) table[k] = (uint8_t)order[k];
    return EC_OK;
}

uint64_t bf16_exp_max_encoded_bytes(uint64_t n, uint32_t chunk) {
    if (!bf_chunk_ok(chunk) || n > kMaxSegSymbols) return 0;
    return bf_layout(n, chunk).esc_at + n;
}

int bf16_exp_encode(const uint8_t table[7], const uint16_t *d_in, uint64_t n, uint32_t chunk, uint8_t *d_out,
                    uint64_t out_cap, uint64_t *d_out_len, uint32_t *d_status, hipStream_t stream) {
    if (!table || !d_out || !d_out_len || (n && !d_in) || !bf_chunk_ok(chunk) || n > kMaxSegSymbols)
        return EC_E_INVAL;
    if (!aligned16(d_in) || !aligned16(d_out)) return EC_E_INVAL;
    for (int i = 0; i < 7; ++i)
        for (int j = 0; j < i; ++j)
            if (table[i] == table[j]) return EC_E_INVAL;
    const BfLayout L = bf_layout(n, chunk);
    if (L.n_chunks > kBfMaxChunks) return EC_E_UNSUPPORTED;
    if (out_cap < L.esc_at) return EC_E_CAPACITY;
    BfArgs a;
    memset(&a, 0, sizeof(a));
    a.in = d_in;
    a.n = n;
    a.out = d_out;
    a.out_cap = out_cap;
    a.out_len = d_out_len;
    a.status = d_status;
    a.sm_at = L.sm_at;
    a.plane_at = L.plane_at;
    a.plane_bytes = L.plane_bytes;
    a.esc_at = L.esc_at;
    a.chunk = chunk;
    a.n_chunks = (uint32_t)L.n_chunks;
    for (int k = 0; k < 7; ++k) a.table[1 + k] = table[k];
    if (L.n_chunks) {
        void *p = nullptr;
        int rc = device_scratch(kScratchBfCounts, L.n_chunks * 4, stream, &p);
        if (rc) return rc;
        a.counts = static_cast<uint32_t *>(p);
        rc = device_scratch(kScratchBfEsc, L.n_chunks * chunk, stream, &p);
        if (rc) return rc;
        a.esc_tmp = static_cast<uint8_t *>(p);
    }
    return hip_rc(launch_bf16_encode(a, stream));
}

int bf16_exp_decode(const uint8_t *d_in, uint64_t in_len, uint16_t *d_out, uint64_t n, uint32_t *d_status,
                    hipStream_t stream) {
    if (!d_in || in_len < kHeaderBytes || (n && !d_out) || n > kMaxSegSymbols) return EC_E_INVAL;
    if (!aligned16(d_in) || !aligned16(d_out)) return EC_E_INVAL;
    BfDecArgs a;
    memset(&a, 0, sizeof(a));
    a.in = d_in;
    a.in_len = in_len;
    a.out = d_out;
    a.n = n;
    a.status = d_status;
    return hip_rc(launch_bf16_decode(a, stream));
}
