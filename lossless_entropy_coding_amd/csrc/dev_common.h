// Device-side helpers and launch interfaces shared by the libec kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ec_internal.h"

namespace ec {

// Compile-time loop: f(std::integral_constant<int, I>) for I = B..E-1, so that
// register arrays indexed by I stay in registers.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Table pointer of segment `seg`, read straight from the kernel-argument
// segment (constant address space).  Indexing the by-value argument with a
// run-time index would make the compiler copy the whole argument block
// (with its 128 pointers) into per-lane scratch memory.
template <class Args>
__device__ __forceinline__ const DevTables *seg_tables(uint32_t seg) {
    typedef __attribute__((address_space(4))) const Args CArgs;
    const CArgs *p = (const CArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    return p->tabs[seg];
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts within
// each row of 16 lanes, then the row broadcasts of lanes 15 and 31 (lanes
// whose DPP source is outside the row, or whose row is masked off, add 0).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return x;
}

// Status bits are OR-ed at device (agent) scope: visible across the eight
// XCDs' separate L2 caches.
__device__ __forceinline__ void or_status(uint32_t *status, uint32_t bits) {
    if (status) __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- launches

struct EncodeArgs {
    const uint8_t *in;
    uint64_t in_stride;
    uint64_t seg_n;
    uint8_t *out;
    uint64_t out_stride;
    uint64_t out_cap;
    uint64_t *out_len;        // [n_seg]
    uint32_t *status;         // [n_seg] or null
    uint32_t *sizes;          // chunk sizes in 16-byte units, one per chunk of the launch
    uint32_t chunk_symbols;
    uint32_t chunks_per_seg;
    uint32_t n_seg;
    uint32_t payload_offset;
    uint32_t sub_at;          // byte offset of sub_end[] in a stream
    uint32_t embed_lengths;
    uint32_t max_len;         // longest code over the launch's codebooks
    uint32_t stage_bytes;     // LDS stage of the staged packer (set at launch)
    uint32_t tables_unread;   // 1: the host never read the tables (device-built); the packers check
                              // each chunk's table for codes longer than kNarrowMaxLen themselves
    uint32_t place_in_pack;   // 1: this pack launch sums the chunk sizes itself and writes chunk_off[],
                              // the header and the index tail (no separate offsets launch)
    uint32_t staged_rows;     // 1: the staged packer packs a chunk that overflows its stage row by row
                              // in the stage itself (the row packer then skips such chunks)
    uint32_t sized;           // 1: sizes come from the caller (a histogram pass made them): no sizes
                              // launch; the packer writes sub_end[] and checks its chunk's size
    const DevTables *tabs[EC_MAX_BATCH];
};

struct DecodeArgs {
    const uint8_t *in;
    uint64_t in_stride;
    uint64_t in_len;          // readable bytes per stream
    uint8_t *out;
    uint64_t out_stride;
    uint64_t seg_n;
    uint32_t *status;         // [n_seg] or null
    uint32_t n_seg;
    uint32_t blocks_per_seg;  // 256-symbol runs per segment
    const DevTables *tabs[EC_MAX_BATCH];
};

// BF16 exponent coding (bf16exp.hip).
struct BfArgs {
    const uint16_t *in;
    uint64_t n;
    uint8_t *out;
    uint64_t out_cap;
    uint64_t *out_len;
    uint32_t *status;         // or null
    uint32_t *counts;         // escapes per chunk (scratch)
    uint8_t *esc_tmp;         // escapes of chunk c staged at esc_tmp + c * chunk (scratch)
    uint64_t sm_at, plane_at, plane_bytes, esc_at;
    uint32_t chunk, n_chunks;
    uint8_t table[8];         // table[1..7]: the exponent of code k
};

struct BfDecArgs {
    const uint8_t *in;
    uint64_t in_len;
    uint16_t *out;
    uint64_t n;
    uint32_t *status;         // or null
};

hipError_t launch_bf16_encode(const BfArgs &a, hipStream_t s);
hipError_t launch_bf16_decode(const BfDecArgs &a, hipStream_t s);

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s);
// Whether an encode with caller-made sizes can run: every chunk then goes
// through the staged packer (codes of up to kNarrowMaxLen bits from tables
// the host has read, chunks of up to four rows).
bool encode_sized_supported(uint32_t chunk_symbols, uint32_t max_len);
hipError_t launch_decode(const DecodeArgs &a, uint32_t codec, uint32_t max_len, hipStream_t s);
// Chunk sizes made by the histogram's pass over the input: for each of n_cb
// codebooks, the size in 16-byte units that an encode with chunk_symbols =
// 16 << vc_log2 gives every chunk (what its sizes launch would write).
constexpr uint32_t kMaxSizeCodebooks = 4;
struct ChunkSizeArgs {
    const DevTables *tabs[kMaxSizeCodebooks];
    uint32_t *sizes;          // [n_cb][n_seg][chunks_per_seg]
    uint32_t n_cb;            // 1..kMaxSizeCodebooks
    uint32_t vc_log2;         // log2 of the 16-byte vectors of a chunk
    uint32_t chunks_per_seg;
};

// Partial-count rows per segment of a histogram launch (uint32 x 256 each),
// without or with chunk sizes.
uint32_t histogram_blocks(uint64_t seg_n, uint32_t n_seg, bool sized = false);
// Whether a histogram launch can also make the chunk sizes for chunks of
// chunk_symbols: a power of two that divides the launch's pieces, with
// every segment a whole number of 16-byte vectors.
bool histogram_can_size(uint64_t seg_n, uint32_t n_seg, uint32_t chunk_symbols);
hipError_t launch_histogram(const uint8_t *in, uint64_t seg_n, uint32_t n_seg, uint64_t in_stride,
                            uint64_t *counts, uint32_t *partial, const ChunkSizeArgs *cs, hipStream_t s);
hipError_t launch_huff_build(const uint64_t *counts, uint32_t n_seg, DevTables *tabs, uint32_t *status,
                             hipStream_t s);
hipError_t launch_huff_tables_from_streams(const uint8_t *in, uint64_t in_stride, uint64_t in_len,
                                           uint32_t n_seg, DevTables *tabs, uint32_t *status, hipStream_t s);
hipError_t launch_pmf_average(const uint64_t *counts, uint32_t n_seg, float *pmf, hipStream_t s);
hipError_t launch_pmf_kl(const uint64_t *p, uint32_t n_seg, const uint64_t *q, uint32_t q_add,
                         float *kl, hipStream_t s);

}  // namespace ec
