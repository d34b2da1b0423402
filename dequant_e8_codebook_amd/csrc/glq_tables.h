// glq_tables.h -- layout of the GLQ_CB_DEVICE decode tables (library-internal).
//
// The codebook is the first 65,536 points of the E8 lattice in the stated
// order ("glq 0.1.1", "How it works", item 1). Decoding index i never reads a
// flat 65536 x 8 table (256-512 KiB, larger than the 160 KiB of LDS of a
// gfx950 CU). It walks three small LDS-resident tables instead:
//
//   i' = (i - 1) mod 2^16          the origin (i = 0) lands on i' = 65535
//   CT[i' >> 4]   (uint16)         chunk table, 16 consecutive indices per chunk:
//                                  e = (first_record << 5) | ls, where ls = log2 of
//                                  the orbit size when orbits are smaller than 16
//                                  (several orbits per chunk), 4 otherwise, 0 for the
//                                  last chunk (one record per slot)
//   rec = OT[(e >> 5) + ((i' & 15) >> ls)]   orbit record, 2 x uint32:
//        word 0 = r_lo | lo_off << 8
//                 r_lo    number of nonzero coordinates among x1..x4 (bits 0-4,
//                         so a shift or bit-field extract by word 0 uses it)
//                 lo_off  byte offset of the block of signed low halves
//        word 1 = q_width | hi_off' << 8   (hi_off' signed, arithmetic shift back)
//                 q_width 4 for half-integer orbits, 0 for integer orbits
//                 hi_off' byte offset of the block of signed high halves, minus
//                         8 * (orbit_start >> r_lo)
//   lo = HT[lo_off + 8 * (i' & (2^r_lo - 1))]
//   hi = HT[hi_off' + 8 * (i' >> r_lo) + 64 * (popcount(i' & (2^q_width - 1)) & 1)]
//
// Why this works: every orbit (points sharing |x|) is 2^nnz (integer) or 128
// (half-integer) consecutive indices whose sign counter j = i' - start counts
// sign patterns over the nonzero coordinates in order, and every orbit start
// is a multiple of min(orbit size, 16) in i' (orbits are sorted by decreasing
// size inside a shell and shells start at multiples of 16). So the low r_lo
// bits of j equal the low bits of i', and j >> r_lo = (i' >> r_lo) -
// (start >> r_lo). For half-integer points the sign of x8 is fixed by the
// parity rule; with q = parity of the signs of x1..x4, the high-half block is
// stored as 24 entries [q = 0: j_hi 0..7 | q = 1: 0..7 | q = 0: 0..7] and the
// orbit's parity constant P is folded into hi_off' (+64 bytes when P = 1).
//
// Half-vector value formats (8 bytes = 4 x 16 bit, coordinate t in bits 16t..):
//   HT_BF16  bf16 of x_t = y_t / 2                     (2 bpw, and the float32 path)
//   HT_A3    int16 2 * y_t                              (stage 1 at 3 bpw)
//   HT_A4    int16 4 * y_t                              (stage 1 at 4 bpw)
//   HT_B4    uint16 0x4340 + y_t                        (stage 2 at 4 bpw)
//   R3       first 256 codebook entries, 8 x uint16 0x4340 + y_t (stage 2 at 3 bpw)
// with y = 2x. 0x4340 is bf16 192.0; in the binade [128, 256) a bf16 bit
// pattern grows by one per unit, so 0x4340 + u is exactly the bf16 of 192 + u
// for |u| < 64. A packed 16-bit add of a stage-1 and a stage-2 half gives
// 0x4340 + u with u = 2 y1 + y2 = 4 v at 3 bpw (k = 1) and u = 4 y1 + y2 = 8 v
// at 4 bpw (k = 2), where v = C[i1] + 2^-k C[i2] is the decoded value.
#pragma once
#include <stdint.h>

namespace glq {

constexpr uint32_t kCodebookSize = 65536;
constexpr uint32_t kChunks = 4096;
constexpr uint32_t kMaxRecords = 1472;
constexpr uint32_t kMaxHalves = 2368;
constexpr uint32_t kBias = 0x4340u;       // bf16(192.0)
constexpr float kBiasValue = 192.0f;

// byte offsets inside the GLQ_CB_DEVICE blob
constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kCtOff = kHeaderBytes;
constexpr uint32_t kCtBytes = kChunks * 2;
constexpr uint32_t kOtOff = kCtOff + kCtBytes;
constexpr uint32_t kOtBytes = kMaxRecords * 8;
constexpr uint32_t kHtBytes = kMaxHalves * 8;
constexpr uint32_t kHtBf16Off = kOtOff + kOtBytes;
constexpr uint32_t kHtA3Off = kHtBf16Off + kHtBytes;
constexpr uint32_t kHtA4Off = kHtA3Off + kHtBytes;
constexpr uint32_t kHtB4Off = kHtA4Off + kHtBytes;
constexpr uint32_t kR3Off = kHtB4Off + kHtBytes;
constexpr uint32_t kR3Bytes = 256 * 16;
constexpr uint32_t kBlobBytes = kR3Off + kR3Bytes;

constexpr uint32_t kMagic0 = 0x43514C47u;  // "GLQC"
constexpr uint32_t kFormatVersion = 0x00020000u;

static_assert(kCtOff % 16 == 0 && kOtOff % 16 == 0 && kHtBf16Off % 16 == 0 &&
              kHtA3Off % 16 == 0 && kHtA4Off % 16 == 0 && kHtB4Off % 16 == 0 && kR3Off % 16 == 0,
              "table alignment");

}  // namespace glq
