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

constexpr int kL1Bits = 11;              // first-level decode table index width
constexpr int kL1Size = 1 << kL1Bits;
constexpr int kL2Size = 2048;            // second-level decode table entries (Huffman)
constexpr int kL2MaxBits = 8;            // bits indexed by one second-level sub-table
constexpr int kNarrowMaxLen = 26;        // codes up to this length use 32-bit encode entries (6-bit length field)

// Decode table entry formats (uint16):
//  QLC level 1   : bits 0-7 symbol, bit 8 set = suffix is not a codeword
//  Huffman L1    : bit 15 clear -> bits 0-7 symbol, bits 8-11 code length (1..11)
//                  bit 15 set   -> long prefix: bits 0-10 base index into l2,
//                                  bits 12-14 (sub-table width - 1)
//  Huffman L2    : bits 0-7 symbol, bits 8-12 code length (12..19); 0 length = deeper code
constexpr uint16_t kQlcInvalid = 0x100;
constexpr uint16_t kL1Long = 0x8000;

// Everything a kernel needs about one codebook, uploaded as one blob.
struct alignas(16) DevTables {
    uint64_t enc64[256];      // code << (64 - len) | len: left-aligned code, any length <= 40
    uint32_t enc32[256];      // code << (32 - len) | len, when max_len <= 26 (0 otherwise)
    uint16_t l1[kL1Size];     // decode level 1
    uint16_t l2[kL2Size];     // decode level 2 (Huffman)
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
int huffman_lengths(const uint64_t *weights, uint32_t n, uint8_t *len_out);

}  // namespace ec
