// Internal layouts shared by the host code and the HIP kernels of libec.
#pragma once

#include <stdint.h>

#include <mutex>

#include "ec.h"

namespace ec {

constexpr uint32_t kMagic = 0x53384345u;  // "EC8S"
constexpr uint16_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 64;
constexpr uint32_t kSub = 256;           // symbols per sub-chunk
constexpr uint32_t kMinChunk = 256;
constexpr uint32_t kMaxChunk = 65536;

constexpr int kL1Bits = 11;              // QLC decode table index width (codes <= 11 bits)
constexpr int kL1Size = 1 << kL1Bits;
constexpr int kHuffBits = 13;            // Huffman decode table index width
constexpr int kHuffSize = 1 << kHuffBits;
constexpr int kNarrowMaxLen = 26;        // codes up to this length use 32-bit encode entries (6-bit length field)

// Decode table entry formats (uint16):
//  QLC (11-bit index)     : bits 0-7 symbol, bit 8 set = suffix is not a codeword
//  Huffman (13-bit index) : bits 0-7 symbol, bits 8-12 code length (1..13);
//                           0 = the code is longer than 13 bits (canonical
//                           limit search)
constexpr uint16_t kQlcInvalid = 0x100;

// Everything a kernel needs about one codebook, uploaded as one blob.
struct alignas(16) DevTables {
    uint64_t enc64[256];      // code << (64 - len) | len: left-aligned code, any length <= 40
    uint32_t enc32[256];      // code << (32 - len) | len, when max_len <= 26 (0 otherwise)
    uint16_t l1[kL1Size];     // QLC decode table
    uint16_t hl1[kHuffSize];  // Huffman decode table
    uint64_t limit[48];       // Huffman: 40-bit left-justified end of codes of length l
    uint64_t first_code[48];  // Huffman: canonical first code of length l
    uint32_t first_idx[48];   // Huffman: position of that code in sorted_sym
    uint8_t sym[256];         // QLC/EG: rank -> byte; Huffman: canonical order -> byte
    uint8_t code_len[256];    // per byte, for embedding in streams
    uint64_t codebook_id;
    uint32_t codec;
    uint32_t max_len;
    uint32_t qlc_lens;        // QLC: 4-bit total code length of area a at bits 4a..4a+3
    int32_t eg_k;
    uint32_t pad[2];
};

}  // namespace ec

// The opaque handle of the C ABI.
struct ec_codebook {
    ec::DevTables host;                 // host copy of the tables
    uint16_t area_size[8];
    uint8_t suffix_bits[8];
    std::mutex mu;                      // guards dev[]
    ec::DevTables *dev[16] = {};        // device copy per device id, uploaded at first use
};

namespace ec {

// host builders (codebook.cpp)
int build_qlc(const uint64_t counts[256], const uint16_t area_size[8], const uint8_t suffix_bits[8],
              ec_codebook **out);
int build_huffman_lengths(const uint8_t code_len[256], ec_codebook **out);
int build_eg(const uint64_t counts[256], int k, ec_codebook **out);
int qlc_optimal_areas(const uint64_t counts[256], uint32_t max_lengths, uint16_t area_size[8],
                      uint8_t suffix_bits[8]);
int huffman_lengths(const uint64_t *weights, uint32_t n, uint8_t *len_out);

}  // namespace ec
