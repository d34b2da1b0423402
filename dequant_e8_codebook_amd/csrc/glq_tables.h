// glq_tables.h -- layout of the GLQ_CB_DEVICE decode tables (library-internal),
// format 3.
//
// The codebook is the first 65,536 points of the E8 lattice in the stated
// order ("glq 0.1.1", "How it works", item 1). Decoding index i never reads a
// flat 65536 x 8 table (256-512 KiB, larger than the 160 KiB of LDS of a
// gfx950 CU). It reads one 4-byte record and two signed half-vectors instead:
//
//   i' = (i - 1) mod 2^16            the origin (i = 0) lands on i' = 65535
//   rec = RT[i' >> 2]                record of the 4-index chunk holding i'
//     bits  0-1   t_lo   width of the low-half window of i' (0..2)
//     bits  5-15  LO     byte offset of the low-half run (a multiple of 32)
//     bits 16-17  T      offset of the high-half window of i' (0..2)
//     bits 21-31  HI     entry index of the high-half run
//   lo = HT[LO / 8 + (i' & (2^t_lo - 1))]            coordinates x1..x4
//   hi = HT[HI + ((i' >> T) & 3)]                    coordinates x5..x8
//
// Why one record per 4 indices suffices: every orbit (points sharing |x|)
// is a run of 2^nnz (integer points) or 128 (half-integer points) indices
// that starts at a multiple of its size within its shell, and every shell
// starts at a multiple of 16 in i'. So a chunk of 4 lies inside one orbit of
// size >= 4, and its sign counters are j0 .. j0 + 3 with j0 a multiple of 4:
// only the two lowest sign bits vary inside a chunk. For integer points they
// flip the first two nonzero coordinates, so the low half takes 2^t_lo values
// (t_lo = number of nonzeros among x1..x4, at most 2) and the high half
// varies with i' >> t_lo. For half-integer points the two lowest bits are
// the signs of x1 and x2 and the parity-fixed sign is that of x4, so the high
// half is constant in a chunk (T = 2, its window then covers two constant
// bits of i' that HI absorbs). Three chunks need their own runs: the two
// chunks of the size-2 orbits (+-2 at one coordinate, two orbits per chunk)
// and the last chunk, which holds the three last codebook points and the
// origin (t_lo = 2, T = 0, runs [l0 l1 l2 0] and [h h h 0]).
//
// Half-vector value formats (8 bytes = 4 x 16 bit, coordinate t in bits 16t..):
//   HT_BF16  bf16 of x_t = y_t / 2          (2 bpw, and the float32 path)
//   HT_T     uint16 0xDA40 + y_t (mod 2^16) (3 and 4 bpw, both stages at 4 bpw)
//   R3       first 256 codebook entries, 8 x uint16 0x8EC0 + y_t (stage 2 at 3 bpw)
// with y = 2x. In the binade [128, 256) a bf16 bit pattern grows by one per
// unit, so 0x4340 + u is exactly the bf16 of 192 + u for |u| < 64. One packed
// 16-bit multiply-add of a stage-1 and a stage-2 half gives it:
//   4 bpw: 4 (0xDA40 + y1) + (0xDA40 + y2) = 5 * 0xDA40 + 4 y1 + y2 = 0x4340 + 8 v
//   3 bpw: 2 (0xDA40 + y1) + (0x8EC0 + y2) = 0x4340 + 2 y1 + y2      = 0x4340 + 4 v
// (mod 2^16), where v = C[i1] + 2^-k C[i2] is the decoded value (k = 2 at
// 4 bpw, 1 at 3 bpw).
#pragma once
#include <stdint.h>

namespace glq {

constexpr uint32_t kCodebookSize = 65536;
constexpr uint32_t kChunks = 16384;               // 4 indices per record
constexpr uint32_t kMaxHalves = 2048;             // HI has 11 bits
constexpr uint32_t kBias = 0x4340u;               // bf16(192.0)
constexpr float kBiasValue = 192.0f;
constexpr uint32_t kHtBase = 0xDA40u;             // 5 * kHtBase = kBias (mod 2^16)
constexpr uint32_t kR3Base = 0x8EC0u;             // 2 * kHtBase + kR3Base = kBias (mod 2^16)
static_assert(((5u * kHtBase) & 0xFFFFu) == kBias && ((2u * kHtBase + kR3Base) & 0xFFFFu) == kBias,
              "packed multiply-add constants");

// byte offsets inside the GLQ_CB_DEVICE blob
constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kRtOff = kHeaderBytes;
constexpr uint32_t kRtBytes = kChunks * 4;
constexpr uint32_t kHtBytes = kMaxHalves * 8;
constexpr uint32_t kHtBf16Off = kRtOff + kRtBytes;
constexpr uint32_t kHtTOff = kHtBf16Off + kHtBytes;
constexpr uint32_t kR3Off = kHtTOff + kHtBytes;
constexpr uint32_t kR3Bytes = 256 * 16;
constexpr uint32_t kBlobBytes = kR3Off + kR3Bytes;

constexpr uint32_t kMagic0 = 0x43514C47u;  // "GLQC"
constexpr uint32_t kFormatVersion = 0x00030000u;

static_assert(kRtOff % 16 == 0 && kHtBf16Off % 16 == 0 && kHtTOff % 16 == 0 && kR3Off % 16 == 0,
              "table alignment");

// record fields
constexpr uint32_t rec_pack(uint32_t t_lo, uint32_t lo_bytes, uint32_t T, uint32_t hi_entry) {
  return t_lo | lo_bytes | (T << 16) | (hi_entry << 21);
}

}  // namespace glq
