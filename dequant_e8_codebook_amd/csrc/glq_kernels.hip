// glq_kernels.hip -- gfx950 kernels and the GPU entry points of the C ABI.
//
// The layer computes y = U^T (s W^) (V x) ("glq 0.1.1", PyPI, "How it works",
// items 1-2): W^ is never materialised by glq_fused_linear; each kernel
// expands 16-bit E8 indices (plus 8/16-bit residual indices at 3/4 bpw,
// "Bit widths") into weights inside the product, as the EntroPack news item
// describes for its GPU decoder (fused symbol decoding and weight
// reconstruction).
//
// Kernels:
//   rht_rows        sign flips + block fast Walsh-Hadamard transform along rows,
//                   float32 in LDS (x~ = V x on inputs, y = U^T z on outputs);
//                   optionally rounds to bf16 and records each row's sum of the
//                   rounded values (needed by the biased 3/4 bpw operands).
//   rht_rows_blk,   the same for 16-byte aligned rows, out of place: rows of
//   rht_rows_reg,   whole blocks of 1024 .. 16384 with one wave per 1024
//   rht_rows_vec    elements (butterflies in registers and DPP lane stages,
//                   one LDS transpose above the wave); a few rows of any width
//                   on 1024 threads; the rest in radix-16 passes through LDS.
//   ep_gemv_k       entropy-coded layers at batch 1: the symbol decode fused
//                   into the product.
//   decode_weights  indices -> W^ (rotated basis) as float32 or bf16.
//   gemv_bf16       m <= 16: one 16-row weight tile per workgroup, 16 waves split
//                   k, bf16 MFMA 16x16x32 with x~ rows as the M side (the few
//                   activation rows are padded to 16) and weights decoded
//                   straight into the B operand registers.
//   gemm8_bf16      m > 16, k a multiple of 64: 256 x 256 output tiles, 8
//                   waves (two per SIMD, 32 weight rows each), x~
//                   double-buffered in LDS, weights decoded per wave straight
//                   into MFMA B operands.
//   gemm_bf16       m > 16, other k: the same tile with 4 waves of 64 rows.
//   gemv_f32        float32 path: exact float32 weights, float32 FMAs.
//   layer_small     m <= 4: the whole layer (both transforms and the
//                   decode-GEMV) in one launch.
//   ep_decode_k     entropy-coded layers: rANS symbol decode and weight
//                   reconstruction, one wave per 64-lane block.
//   gemm_w2_bf16,   entropy-coded layers: the product on decoded bf16 weights
//   gemm_w_bf16_lds, (m > 16: k a multiple of 64 / other k; m <= 16).
//   gemv_w_bf16
//
// Every kernel that decodes first copies its decode tables (glq_tables.h, or
// the entropy-coded layer's symbol tables) from the caller's buffer into LDS.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "glq.h"
#include "glq_tables.h"

namespace glq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- LDS tables
// LDS layout of the decode tables: [RT][HT][R3 at 3 bpw]
constexpr uint32_t kLdsRt = 0;
constexpr uint32_t kLdsHt = kLdsRt + kRtBytes;
constexpr uint32_t kLdsR3 = kLdsHt + kHtBytes;

template <int BPW> struct TabCfg;
template <> struct TabCfg<2> { static constexpr uint32_t ht = kHtBf16Off, r3_bytes = 0; };
template <> struct TabCfg<3> { static constexpr uint32_t ht = kHtTOff, r3_bytes = kR3Bytes; };
template <> struct TabCfg<4> { static constexpr uint32_t ht = kHtTOff, r3_bytes = 0; };

template <int BPW>
constexpr uint32_t lds_table_bytes() { return kLdsR3 + TabCfg<BPW>::r3_bytes; }

// blob offset of LDS table byte pos
template <int BPW>
__device__ __forceinline__ uint32_t table_src(uint32_t pos) {
  return pos < kLdsHt ? kRtOff + pos : pos < kLdsR3 ? TabCfg<BPW>::ht + (pos - kLdsHt) : kR3Off + (pos - kLdsR3);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Copy RT + the value table of this bit width (+ R3 at 3 bpw) into LDS (bytes
// 0 .. lds_table_bytes) with global-to-LDS loads: no registers held, nothing
// waited for here. Run r (1 KiB of the LDS image) is copied by wave r mod the
// wave count, lane i writing its bytes 16 i .. 16 i + 15. The caller waits
// with tables_landed() before the barrier that publishes the tables.
template <int BPW, int NT = 256>
__device__ __forceinline__ void load_tables(uint8_t *, const uint8_t *blob) {
  constexpr uint32_t total = lds_table_bytes<BPW>();
  constexpr uint32_t runs = total / 1024;
  static_assert(total % 1024 == 0 && kLdsHt % 1024 == 0 && kLdsR3 % 1024 == 0, "LDS table runs");
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (uint32_t r = wave; r < runs; r += NT / 64) {
    const uint32_t pos = 1024 * r + 16 * lane;
    __builtin_amdgcn_global_load_lds((glb_void_t *)(blob + table_src<BPW>(pos)), (lds_void_t *)(uintptr_t)(1024 * r),
                                     16, 0, 0);
  }
}

// wait for this wave's vector-memory loads, the table copies included
__device__ __forceinline__ void tables_landed() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// LDS pointers built from absolute addresses. Every kernel that decodes uses
// dynamic LDS only (no static __shared__), so its dynamic region starts at
// offset 0 and the table offsets are compile-time constants that fold into
// the DS instructions' offset field (a pointer to the extern array would add
// its link-time base with a VALU add on every lookup).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const uint16_t lds_u16;
typedef __attribute__((address_space(3))) const u32x2_t lds_u64;
typedef __attribute__((address_space(3))) const u32x4_t lds_u128;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
__device__ __forceinline__ uint32_t lds16(uint32_t addr) {
  return *reinterpret_cast<lds_u16 *>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ uint32_t lds_rd32(uint32_t addr) {
  return *reinterpret_cast<lds_u32 *>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ uint2 lds64(uint32_t addr) {
  const u32x2_t v = *reinterpret_cast<lds_u64 *>(static_cast<uintptr_t>(addr));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 lds128(uint32_t addr) {
  const u32x4_t v = *reinterpret_cast<lds_u128 *>(static_cast<uintptr_t>(addr));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef __attribute__((address_space(3))) uint16_t lds_u16_w;
typedef __attribute__((address_space(3))) float lds_f32_w;
__device__ __forceinline__ void lds_st16(uint32_t addr, uint32_t v) {
  *reinterpret_cast<lds_u16_w *>(static_cast<uintptr_t>(addr)) = static_cast<uint16_t>(v);
}
__device__ __forceinline__ void lds_stf(uint32_t addr, float v) {
  *reinterpret_cast<lds_f32_w *>(static_cast<uintptr_t>(addr)) = v;
}

// i' = i - 1 (mod 2^16) for the two 16-bit indices packed in a word.
__device__ __forceinline__ uint32_t pk_dec16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w) - (u16x2)(1));
}

// Byte offsets (inside HT) of the low and high half-vectors of index i',
// from the record of its chunk (glq_tables.h): the low window is
// bfe(i', 0, t_lo) with t_lo in bits 0-4 of the record, the high window
// bfe(i', T, 2) with T in bits 0-4 of rec >> 16, and (rec >> 16) >> 2 is 8 HI.
__device__ __forceinline__ void rec_offsets(uint32_t ip, uint32_t rec, uint32_t &lo, uint32_t &hi) {
  lo = (rec & 0xFFE0u) + (__builtin_amdgcn_ubfe(ip, 0, rec) << 3);
  const uint32_t wh = rec >> 16;
  hi = (wh >> 2) + (__builtin_amdgcn_ubfe(ip, wh, 2) << 3);
}

// record of index i' = i - 1 mod 2^16 (RT entry i' >> 2 at byte i' & ~3)
__device__ __forceinline__ uint32_t rec_of(uint32_t ip) { return lds_rd32(kLdsRt + (ip & 0xFFFCu)); }

__device__ __forceinline__ uint32_t pk_add16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}

// Stage-1 and stage-2 halves into operand form: 16-bit lanes M * a + b
// (mod 2^16), M = 2 at 3 bpw and 4 at 4 bpw (one packed multiply-add).
// MAD: the multiplier is hidden from the optimiser (an empty asm), which then
// emits one v_pk_mad_u16 instead of a shift and an add (the decode-GEMM with
// partial x~ tiles keeps the shift and add: there the one-instruction form
// cost registers)
template <uint16_t M, bool MAD = true>
__device__ __forceinline__ uint32_t pk_comb(uint32_t a, uint32_t b) {
  uint32_t mm = (uint32_t)M * 0x10001u;
  if constexpr (MAD) asm("" : "+s"(mm));
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) * __builtin_bit_cast(u16x2, mm) +
                                          __builtin_bit_cast(u16x2, b));
}

// Decode one group into 8 x 16-bit operand values, coordinate t in half t of
// the result (uint4 = 8 halves). 2 bpw: bf16 of v. 3/4 bpw: bf16 of 192 + u
// with u = 4 v (3 bpw) or 8 v (4 bpw). ip1 = i1 - 1 mod 2^16; at 4 bpw
// a2 = i2 - 1 mod 2^16 too, at 3 bpw a2 = i2 (a direct table row).
template <int BPW>
__device__ __forceinline__ uint4 decode_ip(uint32_t ip1, uint32_t a2) {
  uint32_t lo, hi;
  rec_offsets(ip1, rec_of(ip1), lo, hi);
  const uint2 a = lds64(kLdsHt + lo);
  const uint2 b = lds64(kLdsHt + hi);
  if constexpr (BPW == 2) {
    (void)a2;
    return make_uint4(a.x, a.y, b.x, b.y);
  } else if constexpr (BPW == 3) {
    const uint4 r = lds128(kLdsR3 + (a2 << 4));
    return make_uint4(pk_comb<2>(a.x, r.x), pk_comb<2>(a.y, r.y), pk_comb<2>(b.x, r.z), pk_comb<2>(b.y, r.w));
  } else {
    uint32_t lo2, hi2;
    rec_offsets(a2, rec_of(a2), lo2, hi2);
    const uint2 c = lds64(kLdsHt + lo2);
    const uint2 d = lds64(kLdsHt + hi2);
    return make_uint4(pk_comb<4>(a.x, c.x), pk_comb<4>(a.y, c.y), pk_comb<4>(b.x, d.x), pk_comb<4>(b.y, d.y));
  }
}

// Same, from plain indices (i1, and i2 of its plane).
template <int BPW>
__device__ __forceinline__ uint4 decode_group(uint32_t i1, uint32_t i2, const uint8_t *) {
  return decode_ip<BPW>((i1 - 1u) & 0xFFFFu, BPW == 4 ? ((i2 - 1u) & 0xFFFFu) : i2);
}

// Decode of 8 groups split into phases, so that the LDS reads of one phase
// are in flight together: p1 the chunk records (and the direct residual rows
// at 3 bpw), p2 the half-vector offsets and reads, p3 the combine into
// operand form (as decode_ip). Each phase takes a range [G0, G1) of the
// groups, so a caller can stagger them. q1 / q2 hold the indices as
// decode_ip takes them.
template <int BPW, bool MAD = true>
struct Dec8 {
  uint32_t R1[8], R2[8];
  uint4 r3[8];
  uint2 va[8], vb[8], vc[8], vd[8];

  template <int G0 = 0, int G1 = 8>
  __device__ __forceinline__ void p1(const uint32_t (&q1)[8], const uint32_t (&q2)[8]) {
#pragma unroll
    for (int g = G0; g < G1; ++g) {
      R1[g] = rec_of(q1[g]);
      if constexpr (BPW == 4) R2[g] = rec_of(q2[g]);
      if constexpr (BPW == 3) r3[g] = lds128(kLdsR3 + (q2[g] << 4));
    }
  }
  template <int G0 = 0, int G1 = 8>
  __device__ __forceinline__ void p2(const uint32_t (&q1)[8], const uint32_t (&q2)[8]) {
#pragma unroll
    for (int g = G0; g < G1; ++g) {
      uint32_t lo, hi;
      rec_offsets(q1[g], R1[g], lo, hi);
      va[g] = lds64(kLdsHt + lo);
      vb[g] = lds64(kLdsHt + hi);
      if constexpr (BPW == 4) {
        uint32_t lo2, hi2;
        rec_offsets(q2[g], R2[g], lo2, hi2);
        vc[g] = lds64(kLdsHt + lo2);
        vd[g] = lds64(kLdsHt + hi2);
      }
    }
  }
  template <int G0 = 0, int G1 = 8>
  __device__ __forceinline__ void p3(uint4 (&out)[8]) {
#pragma unroll
    for (int g = G0; g < G1; ++g) {
      if constexpr (BPW == 2) out[g] = make_uint4(va[g].x, va[g].y, vb[g].x, vb[g].y);
      else if constexpr (BPW == 3)
        out[g] = make_uint4(pk_comb<2, MAD>(va[g].x, r3[g].x), pk_comb<2, MAD>(va[g].y, r3[g].y),
                            pk_comb<2, MAD>(vb[g].x, r3[g].z), pk_comb<2, MAD>(vb[g].y, r3[g].w));
      else
        out[g] = make_uint4(pk_comb<4, MAD>(va[g].x, vc[g].x), pk_comb<4, MAD>(va[g].y, vc[g].y),
                            pk_comb<4, MAD>(vb[g].x, vd[g].x), pk_comb<4, MAD>(vb[g].y, vd[g].y));
    }
  }
  // all phases at once
  __device__ __forceinline__ void run(const uint32_t (&q1)[8], const uint32_t (&q2)[8], uint4 (&out)[8]) {
    p1(q1, q2);
    p2(q1, q2);
    p3(out);
  }
};

// value of one decoded 16-bit operand as the exact float32 v
template <int BPW>
__device__ __forceinline__ float operand_value(uint32_t h16) {
  const float f = __uint_as_float(h16 << 16);
  if constexpr (BPW == 2) return f;
  else if constexpr (BPW == 3) return (f - kBiasValue) * 0.25f;
  else return (f - kBiasValue) * 0.125f;
}

// epilogue factors: z = post * (acc - bias * rowsum(x~)) with post = s (2 bpw),
// s/4 (3 bpw), s/8 (4 bpw) and bias = 0 / 192 / 192
template <int BPW> struct Epi;
template <> struct Epi<2> { static constexpr float bias = 0.0f, mul = 1.0f; };
template <> struct Epi<3> { static constexpr float bias = kBiasValue, mul = 0.25f; };
template <> struct Epi<4> { static constexpr float bias = kBiasValue, mul = 0.125f; };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bf16 bit patterns of two floats (a in bits 0-15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)bf16x2_rne(f, 0.0f); }

__device__ __forceinline__ void store_out(void *y, glq_dtype dt, size_t off, float v) {
  if (dt == GLQ_F32) reinterpret_cast<float *>(y)[off] = v;
  else reinterpret_cast<uint16_t *>(y)[off] = f32_to_bf16_rne(v);
}

__device__ __forceinline__ uint32_t load_idx2(const void *idx2, size_t off, int bpw) {
  if (bpw == 3) return reinterpret_cast<const uint8_t *>(idx2)[off];
  return reinterpret_cast<const uint16_t *>(idx2)[off];
}

// ---------------------------------------------------------------- RHT
// One workgroup per row (grid-stride). Block b = 2^logb; the row holds n/b
// blocks, each transformed in LDS with radix-16 register passes.
template <int R>
__device__ __forceinline__ void fwht_regs(float *v) {
#pragma unroll
  for (int s = 1; s < R; s <<= 1)
#pragma unroll
    for (int m = 0; m < R; m += 2 * s)
#pragma unroll
      for (int t = m; t < m + s; ++t) {
        const float a = v[t], c = v[t + s];
        v[t] = a + c;
        v[t + s] = a - c;
      }
}

// v of lane (lane ^ mask) within the wave, mask a power of two <= 32 known at
// compile time: DPP moves for masks below 16 (quad_perm for 1 and 2; a half-row
// mirror (lane ^ 7) then quad_perm [3,2,1,0] (lane ^ 3) for 4; a row mirror
// (lane ^ 15) then a half-row mirror for 8); for 16 and 32 the gfx950 lane
// swaps, VALU operations that need no trip through the LDS unit.
// v_permlane16_swap(a, b) exchanges the odd 16-lane rows of a with the even
// rows of b, v_permlane32_swap(a, b) the upper half of a with the lower half
// of b; with a = b = v, lane l finds v of lane l ^ 16 (l ^ 32) in the second
// result where bit 4 (bit 5) of l is clear and in the first where it is set.
#define GLQ_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false))
__device__ __forceinline__ float lane_xor(float v, int mask) {
  switch (mask) {
    case 1: return GLQ_DPP(v, 0xB1);
    case 2: return GLQ_DPP(v, 0x4E);
    case 4: return GLQ_DPP(GLQ_DPP(v, 0x141), 0x1B);
    case 8: return GLQ_DPP(GLQ_DPP(v, 0x140), 0x141);
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
    }
  }
}
#undef GLQ_DPP

// LDS layout of every FWHT buffer: one pad float after each 16, so that the
// radix-16 passes (element strides 1, 16, 256, ...) hit distinct banks.
__device__ __forceinline__ int pidx(int i) { return i + (i >> 4); }
__host__ __device__ constexpr size_t padded_floats(size_t n) { return n + n / 16 + 1; }

template <int R>
__device__ __forceinline__ void fwht_pass(float *buf, int b, int lo) {
  const int h = 1 << lo;
  const int nsub = b / R;
  for (int q = threadIdx.x; q < nsub; q += blockDim.x) {
    const int base = (q >> lo) * (h * R) + (q & (h - 1));
    float v[R];
#pragma unroll
    for (int m = 0; m < R; ++m) v[m] = buf[pidx(base + m * h)];
    fwht_regs<R>(v);
#pragma unroll
    for (int m = 0; m < R; ++m) buf[pidx(base + m * h)] = v[m];
  }
}

// The same pass with the stride 2^LO known at compile time, LO a multiple of
// 4. Under pidx's padding, element base + m 2^LO of a thread's R lies at
// pidx(base) + m (2^LO + 2^LO / 16) for LO >= 4 (m 2^LO is a multiple of 16),
// and at pidx(base) + m for LO = 0 (base = q R with R dividing 16, so the R
// elements share one 16-float run): one address register and constant
// offsets instead of a shift and two adds per element.
template <int R, int LO>
__device__ __forceinline__ void fwht_pass_c(float *buf, int b) {
  constexpr int h = 1 << LO;
  constexpr int step = LO == 0 ? 1 : h + h / 16;
  static_assert(LO % 4 == 0 && 16 % R == 0, "stride a multiple of 16, radix dividing 16");
  const int nsub = b / R;
  for (int q = threadIdx.x; q < nsub; q += blockDim.x) {
    float *p = buf + pidx((q >> LO) * (h * R) + (q & (h - 1)));
    float v[R];
#pragma unroll
    for (int m = 0; m < R; ++m) v[m] = p[m * step];
    fwht_regs<R>(v);
#pragma unroll
    for (int m = 0; m < R; ++m) p[m * step] = v[m];
  }
}

template <int R>
__device__ __forceinline__ void fwht_pass_at(float *buf, int b, int lo) {
  switch (lo) {
    case 0: fwht_pass_c<R, 0>(buf, b); break;
    case 4: fwht_pass_c<R, 4>(buf, b); break;
    case 8: fwht_pass_c<R, 8>(buf, b); break;
    case 12: fwht_pass_c<R, 12>(buf, b); break;
    default: fwht_pass<R>(buf, b, lo); break;
  }
}

__device__ __forceinline__ float load_elem(const void *p, glq_dtype dt, size_t off) {
  if (dt == GLQ_F32) return reinterpret_cast<const float *>(p)[off];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[off] << 16);
}

__global__ void __launch_bounds__(256)
rht_rows(const void *in, glq_dtype in_dt, void *out, glq_dtype out_dt, int64_t rows, int64_t n,
         int logb, const int8_t *signs, int transpose, float *rowsum) {
  extern __shared__ float buf[];
  __shared__ float red[256 / 64];
  const int b = 1 << logb;
  const float inv = 1.0f / sqrtf((float)b);   // exact for even logb
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    float rs = 0.0f;
    for (int64_t blk = 0; blk < n; blk += b) {
      const size_t base = (size_t)row * n + blk;
      __syncthreads();
      for (int i = threadIdx.x; i < b; i += blockDim.x) {
        float v = load_elem(in, in_dt, base + i);
        if (!transpose) v *= (float)signs[blk + i];
        buf[pidx(i)] = v;
      }
      __syncthreads();
      int lo = 0;
      for (; lo + 4 <= logb; lo += 4) { fwht_pass<16>(buf, b, lo); __syncthreads(); }
      switch (logb - lo) {
        case 1: fwht_pass<2>(buf, b, lo); break;
        case 2: fwht_pass<4>(buf, b, lo); break;
        case 3: fwht_pass<8>(buf, b, lo); break;
        default: break;
      }
      __syncthreads();
      for (int i = threadIdx.x; i < b; i += blockDim.x) {
        float v = buf[pidx(i)] * inv;
        if (transpose) v *= (float)signs[blk + i];
        if (out_dt == GLQ_F32) {
          reinterpret_cast<float *>(out)[base + i] = v;
          rs += v;
        } else {
          const uint16_t hb = f32_to_bf16_rne(v);
          reinterpret_cast<uint16_t *>(out)[base + i] = hb;
          rs += __uint_as_float((uint32_t)hb << 16);
        }
      }
    }
    if (rowsum) {
      for (int off = 32; off > 0; off >>= 1) rs += __shfl_xor(rs, off);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = rs;
      __syncthreads();
      if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
        rowsum[row] = t;
      }
      __syncthreads();
    }
  }
}

// Vectorised RHT: one workgroup (256 threads) per row, the whole row in LDS
// as float32 (n % 8 == 0, n <= 32768). Each thread moves 8-element pieces
// with 16-byte loads, issued 4 at a time before any LDS write; the row sum of
// the (rounded) outputs is reduced in the workgroup, so it is deterministic.
constexpr int RV_MAX = 32768;

template <bool IN_BF16>
__device__ __forceinline__ void rv_load_piece(const void *in, size_t e0, float (&v)[8]) {
  if constexpr (IN_BF16) {
    const uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(in) + e0);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = __uint_as_float(w[t] << 16);
      v[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(in) + e0);
    const float4 b = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(in) + e0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__device__ __forceinline__ void rv_signs(const int8_t *signs, int64_t i0, float (&sg)[8]) {
  const uint2 u = *reinterpret_cast<const uint2 *>(signs + i0);
#pragma unroll
  for (int t = 0; t < 8; ++t) sg[t] = (float)(int8_t)(((t < 4 ? u.x : u.y) >> (8 * (t & 3))) & 0xFF);
}

// Pieces of 8 consecutive inputs as loaded (bf16: one 16-byte word; float32:
// two), kept packed until they are written to LDS.
template <bool IN_BF16> struct RvRaw { uint4 a, b; };

template <bool IN_BF16>
__device__ __forceinline__ void rv_fetch(const void *in, size_t e0, RvRaw<IN_BF16> &r) {
  if constexpr (IN_BF16) {
    r.a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(in) + e0);
  } else {
    r.a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(in) + e0);
    r.b = *reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(in) + e0 + 4);
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void rv_unpack(const RvRaw<IN_BF16> &r, float (&v)[8]) {
  if constexpr (IN_BF16) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = __uint_as_float(w[t] << 16);
      v[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = __uint_as_float(w[t]);
  }
}

__device__ __forceinline__ float rv_sign(uint2 u, int t) {
  return (float)(int8_t)(((t < 4 ? u.x : u.y) >> (8 * (t & 3))) & 0xFF);
}

// Rows of n (multiple of 8) through LDS radix-16 passes, 256 threads per row,
// grid-stride over rows. Thread t owns pieces t, t + 256, ... (PT at most) of
// every row. The next row's pieces are loaded into registers right after the
// current row is written to LDS, so they arrive during its passes and
// stores; the signs (the same for every row) are loaded once, packed.
template <bool IN_BF16, bool OUT_BF16, bool TRANSPOSE, int PT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PT == 8 && IN_BF16 ? 3 : 1)))
rht_rows_vec(const void *in, void *out, int64_t rows, int64_t n, int logb, const int8_t *signs,
             float *rowsum) {
  extern __shared__ float buf[];
  __shared__ float red[4];
  const int b = 1 << logb;
  const float inv = 1.0f / sqrtf((float)b);   // exact for even logb
  const int pieces = (int)(n >> 3);
  const int tid = threadIdx.x;
  uint2 sgp[PT];
  RvRaw<IN_BF16> raw[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int pc = min(tid + 256 * u, pieces - 1);     // clamped: pieces past n are not used
    sgp[u] = *reinterpret_cast<const uint2 *>(signs + 8 * (int64_t)pc);
  }
  // Up to 4 pieces a thread: the factor of each element (the same for every
  // row) as floats once, the sign before the transform or sign / sqrt(b)
  // after it (transposed). Passes with compile-time strides up to 4 pieces,
  // and at 8 for bf16 input under a 3-waves-per-SIMD register cap (the
  // kernel attribute): uncapped they take 175 registers, one resident wave
  // per SIMD fewer than the 167 of runtime strides. Float32 input at 8
  // pieces (198 registers either way) keeps runtime strides.
  constexpr bool SGF = PT <= 4;
  float sgf[SGF ? PT : 1][8];
  if constexpr (SGF) {
#pragma unroll
    for (int u = 0; u < PT; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) sgf[u][t] = TRANSPOSE ? rv_sign(sgp[u], t) * inv : rv_sign(sgp[u], t);
  }
  int64_t row = blockIdx.x;
  if (row < rows) {
#pragma unroll
    for (int u = 0; u < PT; ++u) rv_fetch<IN_BF16>(in, (size_t)row * n + 8 * (size_t)min(tid + 256 * u, pieces - 1), raw[u]);
  }
  for (; row < rows; row += gridDim.x) {
    const size_t base = (size_t)row * n;
    __syncthreads();                           // previous row's readers are done with buf
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int pc = tid + 256 * u;
      if (pc < pieces) {
        float v[8];
        rv_unpack<IN_BF16>(raw[u], v);
        float *pp = buf + pidx(8 * pc);                // a piece never crosses a 16-float run
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          float f = 1.0f;
          if constexpr (!TRANSPOSE) f = SGF ? sgf[SGF ? u : 0][t] : rv_sign(sgp[u], t);
          pp[t] = TRANSPOSE ? v[t] : v[t] * f;
        }
      }
    }
    if (row + gridDim.x < rows) {              // next row, in flight during this row's passes
      const size_t nb = base + (size_t)gridDim.x * n;
#pragma unroll
      for (int u = 0; u < PT; ++u) rv_fetch<IN_BF16>(in, nb + 8 * (size_t)min(tid + 256 * u, pieces - 1), raw[u]);
    }
    __syncthreads();
    int lo = 0;
    if constexpr (SGF || (PT == 8 && IN_BF16)) {
      for (; lo + 4 <= logb; lo += 4) { fwht_pass_at<16>(buf, (int)n, lo); __syncthreads(); }
      switch (logb - lo) {
        case 1: fwht_pass_at<2>(buf, (int)n, lo); break;
        case 2: fwht_pass_at<4>(buf, (int)n, lo); break;
        case 3: fwht_pass_at<8>(buf, (int)n, lo); break;
        default: break;
      }
    } else {                                   // float32 rows of 8 pieces, rows of 16: runtime strides
      for (; lo + 4 <= logb; lo += 4) { fwht_pass<16>(buf, (int)n, lo); __syncthreads(); }
      switch (logb - lo) {
        case 1: fwht_pass<2>(buf, (int)n, lo); break;
        case 2: fwht_pass<4>(buf, (int)n, lo); break;
        case 3: fwht_pass<8>(buf, (int)n, lo); break;
        default: break;
      }
    }
    __syncthreads();
    float rs = 0.0f;
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int pc = tid + 256 * u;
      if (pc < pieces) {
        float v[8];
        const float *pp = buf + pidx(8 * pc);
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = pp[t];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if constexpr (TRANSPOSE && SGF) v[t] *= sgf[SGF ? u : 0][t];
          else {
            v[t] *= inv;
            if (TRANSPOSE) v[t] *= rv_sign(sgp[u], t);
          }
        }
        if constexpr (OUT_BF16) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t hh = bf16x2_rne(v[2 * t], v[2 * t + 1]);
            const uint16_t h0 = (uint16_t)hh, h1 = (uint16_t)(hh >> 16);
            w[t] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            rs += __uint_as_float((uint32_t)h0 << 16) + __uint_as_float((uint32_t)h1 << 16);
          }
          *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + base + 8 * (size_t)pc) =
              make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          float *o = reinterpret_cast<float *>(out) + base + 8 * (size_t)pc;
          reinterpret_cast<float4 *>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
          reinterpret_cast<float4 *>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
#pragma unroll
          for (int t = 0; t < 8; ++t) rs += v[t];
        }
      }
    }
    if (rowsum) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) rs += lane_xor(rs, off);   // DPP / lane swaps, no LDS
      if ((tid & 63) == 0) red[tid >> 6] = rs;
      __syncthreads();
      if (tid == 0) rowsum[row] = red[0] + red[1] + red[2] + red[3];
    }
  }
}

// row sums of a bf16 [rows][n] array (x already rotated, biased operands need them)
__global__ void __launch_bounds__(256)
row_sums_bf16(const uint16_t *x, int64_t rows, int64_t n, float *rowsum) {
  __shared__ float red[4];
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    float rs = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
      rs += __uint_as_float((uint32_t)x[(size_t)row * n + i] << 16);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) rs += lane_xor(rs, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = rs;
    __syncthreads();
    if (threadIdx.x == 0) rowsum[row] = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
  }
}


// Block FWHT over bits 0 .. logb - 1 of the flat index of 64 NW E elements
// (E = 1, 2, 4, 8, 16 per thread, NW = 4, 8 or 16 waves; 2^logb <= 64 NW E)
// held E per thread. On entry thread t holds elements E t + i in v[i]. The low
// L = log2 E + 6 bits are transformed in registers and across the lanes of the
// wave; when logb > L the values pass once through LDS (buf, 64 NW E + 64
// floats; a pad of 4 floats per 2^L elements keeps the reads conflict-free)
// and the remaining log2 NW bits are transformed the same way. Afterwards
// thread t holds element ly_elem<E, NW>(t, i, transposed) in v[i]: with
// e = lo + 2^L hi, either (E < NW) LPC = NW / E lanes share a column lo, lane
// sub of them holding hi = sub E + i, or (E >= NW) a thread holds the NW
// elements of each of its E / NW columns lo = t + 64 NW c, i = NW c + hi.
// Unscaled: (a, b) -> (a + b, a - b) at every stage.
template <int E, int NW = 16> struct LyF {
  static constexpr int LE = E == 1 ? 0 : E == 2 ? 1 : E == 4 ? 2 : E == 8 ? 3 : 4;
  static constexpr int L = LE + 6;
  static constexpr int WB = NW == 1 ? 0 : NW == 2 ? 1 : NW == 4 ? 2 : NW == 8 ? 3 : 4;
  static constexpr int LPC = E < NW ? NW / E : 1;  // lanes per column after the transpose
  static constexpr int CPT = E < NW ? 1 : E / NW;  // columns per thread after the transpose
};

template <int E, int NW = 16>
__device__ __forceinline__ int ly_elem(int tid, int i, bool transposed) {
  using F = LyF<E, NW>;
  if (!transposed) return E * tid + i;
  if constexpr (E < NW) {
    const int lo = tid / F::LPC, sub = tid % F::LPC;
    return lo + ((sub * E + i) << F::L);
  } else {
    return tid + 64 * NW * (i / NW) + ((i % NW) << F::L);
  }
}

template <int E>
__device__ __forceinline__ void ly_stage_regs(float (&v)[E], int s) {
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (!(i & (1 << s))) {
      const float a = v[i], b = v[i + (1 << s)];
      v[i] = a + b;
      v[i + (1 << s)] = a - b;
    }
}

// one butterfly stage across lane pairs (lane, lane ^ mask): the lower lane
// keeps a + b, the upper one a - b, as o + (+-1) v in one exact fma
template <int E>
__device__ __forceinline__ void ly_stage_lanes(float (&v)[E], int mask, bool upper) {
  const float sg = upper ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = fmaf(v[i], sg, lane_xor(v[i], mask));
}

// One butterfly stage across lane bit 4 (R16) or lane bit 5 for register
// pairs (a, b): the lane swap (16-lane rows, or 32-lane halves) exchanges the
// odd rows of a with the even rows of b, after which every lane holds both
// members of one butterfly pair in its two results (a pair of a in the even
// rows, a pair of b in the odd ones). The butterflies run in registers, and
// the same swap of the sums and differences puts every result back in place:
// four operations per two elements instead of a copy, a swap, a select and an
// fma per element.
template <int E, bool R16>
__device__ __forceinline__ void ly_stage_swap(float (&v)[E]) {
  static_assert(E >= 2 && E % 2 == 0, "register pairs");
#pragma unroll
  for (int p = 0; p < E; p += 2) {
    const auto r = R16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v[p]), __float_as_uint(v[p + 1]), false, false)
                       : __builtin_amdgcn_permlane32_swap(__float_as_uint(v[p]), __float_as_uint(v[p + 1]), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    const float sum = a + b, dif = a - b;
    const auto t = R16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(sum), __float_as_uint(dif), false, false)
                       : __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(dif), false, false);
    v[p] = __uint_as_float(t[0]);
    v[p + 1] = __uint_as_float(t[1]);
  }
}

// The stages above the wave (labels L .. logb - 1, logb > L): an LDS transpose
// to the layout of ly_elem(., ., true), then the butterflies there.
template <int E, int NW>
__device__ __forceinline__ void ly_fwht_cross(float (&v)[E], float *buf, int logb, int tid) {
  using F = LyF<E, NW>;
  constexpr int LE = F::LE, L = F::L;
  {
    float *w = buf + E * tid + 4 * (tid >> 6);         // element E tid + i at e + 4 (e >> L)
    if constexpr (E >= 4) {
#pragma unroll
      for (int i = 0; i < E; i += 4) *reinterpret_cast<float4 *>(w + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) w[i] = v[i];
    }
  }
  __syncthreads();
  if constexpr (E < NW) {
    const int lo = tid / F::LPC, sub = tid % F::LPC;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int hi = sub * E + i;
      v[i] = buf[lo + (hi << L) + 4 * hi];
    }
#pragma unroll
    for (int h = 0; h < F::WB; ++h) {
      if (L + h >= logb) break;
      if (h < LE) ly_stage_regs<E>(v, h);
      else ly_stage_lanes<E>(v, 1 << (h - LE), (sub >> (h - LE)) & 1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int hi = i % NW;
      v[i] = buf[tid + 64 * NW * (i / NW) + (hi << L) + 4 * hi];
    }
#pragma unroll
    for (int h = 0; h < F::WB; ++h) {
      if (L + h >= logb) break;
      ly_stage_regs<E>(v, h);
    }
  }
}

// FULL: the block is all 64 NW E elements (logb = L + log2 NW), so that every
// stage runs and none is tested at run time.
template <int E, int NW = 16, bool FULL = false>
__device__ __forceinline__ bool ly_fwht(float (&v)[E], float *buf, int logb_rt, int tid) {
  using F = LyF<E, NW>;
  constexpr int LE = F::LE, L = F::L;
  const int logb = FULL ? L + F::WB : logb_rt;
  const int lane = tid & 63;
#pragma unroll
  for (int s = 0; s < LE; ++s)
    if (s < logb) ly_stage_regs<E>(v, s);
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    if (LE + s < logb) {
      if constexpr (E >= 2) {
        if (s == 4) { ly_stage_swap<E, true>(v); continue; }
        if (s == 5) { ly_stage_swap<E, false>(v); continue; }
      }
      ly_stage_lanes<E>(v, 1 << s, (lane >> s) & 1);
    }
  }
  if (logb <= L) return false;
  ly_fwht_cross<E, NW>(v, buf, logb, tid);
  return true;
}


__device__ __forceinline__ int ly_e(int count) {    // elements per thread for count <= 16384 elements
  int e = 1;
  while (e * 1024 < count) e <<= 1;
  return e;
}

// Element (r, e) of x~ (r < 16 activation rows, e < k, k a multiple of 256)
// in the layout the small-batch GEMV reads its MFMA 16x16x32 A operands in:
// for chunk c (32 groups of 8 elements) and step s (0..7) one KiB holds lane
// l = j + 16 q's 16 bytes, the 8 elements of group 32 c + 8 q + s of row j.
// A wave then loads each operand as one contiguous KiB instead of 16 rows x
// 64 bytes (16 cache lines), which bound the GEMV's load phase.
__device__ __forceinline__ size_t tile16_index(int64_t r, int e) {
  const int g = e >> 3;
  return ((size_t)((((g >> 5) << 3) + (g & 7)) * 64 + (int)r + 16 * ((g >> 3) & 3)) << 3) + (e & 7);
}

// RHT of rows of length n <= 16384 (n % 8 == 0, 16-byte aligned rows and
// pointers, in != out): one row per workgroup of 64 NW threads (grid-stride),
// the block FWHT in registers and lane exchanges (ly_fwht).
// Raw loads of the thread's E consecutive inputs from element e0 of a row
// (zeros past n), unpacked by rr_unpack: split so that the loads of the next
// row can be in flight while the current one is transformed.
template <int E, bool IN_BF16> struct RrRaw {
  static constexpr int W = IN_BF16 ? (E + 1) / 2 : E;
  uint32_t w[W];
};

template <int E, bool IN_BF16>
__device__ __forceinline__ void rr_fetch(const void *in, size_t base, int e0, int n, RrRaw<E, IN_BF16> &r) {
  bool whole = e0 + E <= n;
  if constexpr (E == 1) whole = false;
  if (whole) {
    if constexpr (IN_BF16) {
      const uint16_t *p = reinterpret_cast<const uint16_t *>(in) + base + e0;
      if constexpr (E == 2) r.w[0] = *reinterpret_cast<const uint32_t *>(p);
      else if constexpr (E == 4) { const uint2 u = *reinterpret_cast<const uint2 *>(p); r.w[0] = u.x; r.w[1] = u.y; }
      else {
#pragma unroll
        for (int c = 0; c < E / 8; ++c) {
          const uint4 u = *reinterpret_cast<const uint4 *>(p + 8 * c);
          r.w[4 * c] = u.x; r.w[4 * c + 1] = u.y; r.w[4 * c + 2] = u.z; r.w[4 * c + 3] = u.w;
        }
      }
    } else {
      const uint32_t *p = reinterpret_cast<const uint32_t *>(in) + base + e0;
      if constexpr (E == 2) { const uint2 u = *reinterpret_cast<const uint2 *>(p); r.w[0] = u.x; r.w[1] = u.y; }
      else if constexpr (E >= 4) {
#pragma unroll
        for (int c = 0; c < E / 4; ++c) {
          const uint4 u = *reinterpret_cast<const uint4 *>(p + 4 * c);
          r.w[4 * c] = u.x; r.w[4 * c + 1] = u.y; r.w[4 * c + 2] = u.z; r.w[4 * c + 3] = u.w;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < RrRaw<E, IN_BF16>::W; ++i) r.w[i] = 0u;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = e0 + i;
      if (e < n) {
        if constexpr (IN_BF16) r.w[i >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(in)[base + e] << (16 * (i & 1));
        else r.w[i] = reinterpret_cast<const uint32_t *>(in)[base + e];
      }
    }
  }
}

template <int E, bool IN_BF16>
__device__ __forceinline__ void rr_unpack(const RrRaw<E, IN_BF16> &r, float (&v)[E]) {
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if constexpr (IN_BF16) v[i] = __uint_as_float(((r.w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16);
    else v[i] = __uint_as_float(r.w[i]);
  }
}



// FULL: the row is one block of all 64 NW E elements (n = 2^logb = 64 NW E),
// so every FWHT stage runs (none tested at run time) and every element is in
// the row (no bounds test per store).
template <int E, int NW, bool IN_BF16, bool OUT_BF16, bool TRANSPOSE, bool TILE16, bool FULL>
__device__ __forceinline__ void rr_rows(const void *in, void *out, int64_t rows, int n, int logb,
                                        const int8_t *signs, float *rowsum, float *buf, float *red) {
  const int tid = threadIdx.x;
  const int e0 = E * tid;
  const float inv = 1.0f / sqrtf((float)(1 << logb));
  // signs of this thread's elements before (sign then FWHT) or after the
  // transform (FWHT then sign, folded with 1 / sqrt(b): an exact product);
  // the element map is the same for every row
  const bool trx = FULL || logb > LyF<E, NW>::L;
  float sg[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = TRANSPOSE ? ly_elem<E, NW>(tid, i, trx) : e0 + i;
    sg[i] = (FULL || e < n) ? (float)signs[e] : 0.0f;
    if (TRANSPOSE) sg[i] *= inv;
  }
  RrRaw<E, IN_BF16> raw;
  if ((int64_t)blockIdx.x < rows) rr_fetch<E, IN_BF16>(in, (size_t)blockIdx.x * n, e0, n, raw);
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const size_t base = (size_t)row * n;
    float v[E];
    rr_unpack<E, IN_BF16>(raw, v);
    if (row + gridDim.x < rows) rr_fetch<E, IN_BF16>(in, base + (size_t)gridDim.x * n, e0, n, raw);   // next row
    if (!TRANSPOSE) {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] *= sg[i];
    }
    __syncthreads();                                 // the previous row is out of buf and red
    const bool tr = ly_fwht<E, NW, FULL>(v, buf, logb, tid);
    float rs = 0.0f;
    float x[E];
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = v[i] * (TRANSPOSE ? sg[i] : inv);
    if constexpr (OUT_BF16) {                        // round to bf16, two at a time
#pragma unroll
      for (int i = 0; i < E; i += 2) {
        const uint32_t hh = bf16x2_rne(x[i], i + 1 < E ? x[i + 1] : 0.0f);
        x[i] = __uint_as_float(hh << 16);
        if (i + 1 < E) x[i + 1] = __uint_as_float(hh & 0xFFFF0000u);
      }
    }
    if (!TILE16 && !tr && E >= 2 && e0 + E <= n) {
      // untransposed: the thread's E consecutive outputs in vector stores
      if constexpr (OUT_BF16) {
        uint32_t w[E / 2 > 0 ? E / 2 : 1];
#pragma unroll
        for (int i = 0; i + 1 < E; i += 2) w[i / 2] = (__float_as_uint(x[i]) >> 16) | (__float_as_uint(x[i + 1]) & 0xFFFF0000u);
        uint16_t *o = reinterpret_cast<uint16_t *>(out) + base + e0;
        if constexpr (E == 2) *reinterpret_cast<uint32_t *>(o) = w[0];
        else if constexpr (E == 4) *reinterpret_cast<uint2 *>(o) = make_uint2(w[0], w[1]);
        else {
#pragma unroll
          for (int c = 0; c < E / 8; ++c)
            *reinterpret_cast<uint4 *>(o + 8 * c) = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
        }
      } else {
        float *o = reinterpret_cast<float *>(out) + base + e0;
        if constexpr (E == 2) *reinterpret_cast<float2 *>(o) = make_float2(x[0], x[1]);
        else if constexpr (E >= 4) {
#pragma unroll
          for (int c = 0; c < E / 4; ++c)
            *reinterpret_cast<float4 *>(o + 4 * c) = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
        }
      }
#pragma unroll
      for (int i = 0; i < E; ++i) rs += x[i];
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int e = ly_elem<E, NW>(tid, i, tr);
        if (FULL || e < n) {
          const size_t o = TILE16 ? tile16_index(row, e) : base + e;
          if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(out)[o] = (uint16_t)(__float_as_uint(x[i]) >> 16);
          else reinterpret_cast<float *>(out)[o] = x[i];
          rs += x[i];
        }
      }
    }
    if (rowsum) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) rs += lane_xor(rs, off);
      if ((tid & 63) == 0) red[tid >> 6] = rs;
      __syncthreads();
      if (tid == 0) {
        float t = 0.0f;
        for (int w = 0; w < NW; ++w) t += red[w];
        rowsum[row] = t;
      }
    }
  }
}

template <bool IN_BF16, bool OUT_BF16, bool TRANSPOSE, int NW, bool TILE16 = false>
__global__ void __launch_bounds__(64 * NW)
rht_rows_reg(const void *in, void *out, int64_t rows, int n, int logb, const int8_t *signs, float *rowsum) {
  extern __shared__ __attribute__((aligned(16))) float rr_buf[];   // 64 NW E + 64 floats
  __shared__ float red[NW];
  int e = 1;
  while (e * 64 * NW < n) e <<= 1;
#define GLQ_RR(E_)                                                                                          \
  do {                                                                                                      \
    if (n == 64 * NW * (E_) && logb == LyF<E_, NW>::L + LyF<E_, NW>::WB)                                    \
      rr_rows<E_, NW, IN_BF16, OUT_BF16, TRANSPOSE, TILE16, true>(in, out, rows, n, logb, signs, rowsum, rr_buf, red); \
    else                                                                                                    \
      rr_rows<E_, NW, IN_BF16, OUT_BF16, TRANSPOSE, TILE16, false>(in, out, rows, n, logb, signs, rowsum, rr_buf, red); \
  } while (0)
  switch (e) {
    case 1: GLQ_RR(1); break;
    case 2: GLQ_RR(2); break;
    case 4: GLQ_RR(4); break;
    case 8: GLQ_RR(8); break;
    default: GLQ_RR(16); break;
  }
#undef GLQ_RR
}

// RHT of rows of nb blocks of B = 1024 NW elements (n = nb B, B the Hadamard
// block, nb NW <= 16): one workgroup of nb NW waves per row (grid-stride over
// rows), NW waves per block with 16 elements per lane, the FWHT over each
// wave's 1024 elements in registers and lane exchanges (rb_fwht_wave: no
// LDS), then for NW > 1 one LDS transpose for the top log2 NW bits
// (ly_fwht_cross) and one back, so that loads and stores are whole 16-byte
// vectors. It replaces the LDS radix-16 kernel on rows of several blocks
// (3072 = 3 x 1024, 12288 = 3 x 4096), whose three to four LDS passes per
// element held it to about 3 TB/s. The next row's inputs are in flight during
// the current row's transform; the row sum of the rounded outputs is reduced
// over the workgroup (deterministic).
//
// Labels: thread t of a block, register i carries label p = 16 t + i, which
// stands for element rb_elem(p) of the block: label bits 0..2 are element
// bits 0..2, label bit 3 is element bit 9, label bits 4..9 (the lane l)
// are element bits 3..8 after the lane relabelling rb_ell, and bits 10 and
// up (the wave) are the same. Lane l of a wave then holds elements
// 8 rb_ell(l) + 0..7 and 512 + 8 rb_ell(l) + 0..7 of its 1024-element chunk,
// so each 16-byte load or store of the wave covers one contiguous KiB.
//
// The lane stages of rb_fwht_wave pair lanes l and l ^ m for m = 1, 2, 7, 8:
// each partner read is a single DPP permutation (quad_perm for 1 and 2, the
// half-row mirror for 7, a rotation by 8 within 16-lane rows for 8), folded
// into one fused multiply-add per element. Stage j transforms bit j of
// rb_ell(l) (its pairs differ in exactly that bit), which makes the four
// stages the Hadamard transform over element bits 3..6. The lower member of
// a pair (bit j of rb_ell(l) clear) keeps a + b, the upper one a - b instead
// of b - a: the upper lane's value is then the negated result, a factor
// rb_sgn(l) = (-1)^popcount(rb_ell(l) & 15) that every later stage carries
// along unchanged (partners share it) and the output scale removes.
__device__ __forceinline__ int rb_ell(int l) { return l ^ (((l >> 2) & 1) * 3); }
__device__ __forceinline__ float rb_sgn(int l) { return (__popc(rb_ell(l) & 15) & 1) ? -1.0f : 1.0f; }
__device__ __forceinline__ int rb_elem(int p) {
  return (p & ~1023) | (p & 7) | (((p >> 3) & 1) << 9) | (rb_ell((p >> 4) & 63) << 3);
}

// One lane stage on 16 registers: v[i] += s * v[i] of the partner lane, the
// partner read by the DPP control CTRL of a v_fmac_f32_dpp (one VALU
// operation per element; the compiler does not fold a DPP move into a
// multiply-add). The leading s_nop gives the two wait states a DPP read needs
// after a VALU write of its source, which the compiler cannot see through the
// asm; inside the block each instruction reads its own register only.
#define RB_FMAC16(CTRL, S)                                                                                  \
  asm volatile("s_nop 1\n\t"                                                                                \
               "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
               "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
               "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
               "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
               "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
               "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
               "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf"                            \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),         \
                 "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]),     \
                 "+v"(v[14]), "+v"(v[15])                                                                    \
               : "v"(S))

// The FWHT over a wave's 1024 labels (E = 16 registers a lane): registers,
// then the four DPP lane stages, then lane bits 4 and 5 by lane swaps.
// Lane bits 4 and 5 (element bits 7 and 8) without the swap back: register
// pairs (p, p + 8) trade lane bit 4, then lane bit 5, for register bit 3, and
// the butterfly results stay where the trade left them. Afterwards register
// bit 3 holds element bit 8, lane bit 5 element bit 7 and lane bit 4 element
// bit 9 (rb_elem_out); register bits 0..2 are still element bits 0..2, so a
// lane's 8 registers of one half are 8 consecutive elements.
template <bool R16>
__device__ __forceinline__ void rb_stage_swap_keep(float (&v)[16]) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const auto r = R16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v[p]), __float_as_uint(v[p + 8]), false, false)
                       : __builtin_amdgcn_permlane32_swap(__float_as_uint(v[p]), __float_as_uint(v[p + 8]), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    v[p] = a + b;
    v[p + 8] = a - b;
  }
}

// element of register i of lane l after rb_fwht_wave<., true>
__device__ __forceinline__ int rb_elem_out(int l, int i) {
  return (i & 7) | ((rb_ell(l) & 15) << 3) | (((l >> 5) & 1) << 7) | (((i >> 3) & 1) << 8) | (((l >> 4) & 1) << 9);
}

template <int FIRST = 0, bool KEEP = false>
__device__ __forceinline__ void rb_fwht_wave(float (&v)[16], int lane) {
  // FIRST = 1: the caller has done register stage 0 (element bit 0);
  // KEEP: the last two stages leave the layout of rb_elem_out
#pragma unroll
  for (int s = FIRST; s < 4; ++s) ly_stage_regs<16>(v, s);
  const int ell = rb_ell(lane);
  const float s0 = (ell & 1) ? -1.0f : 1.0f, s1 = (ell & 2) ? -1.0f : 1.0f;
  const float s2 = (ell & 4) ? -1.0f : 1.0f, s3 = (ell & 8) ? -1.0f : 1.0f;
  RB_FMAC16("quad_perm:[1,0,3,2]", s0);   // lane ^ 1
  RB_FMAC16("quad_perm:[2,3,0,1]", s1);   // lane ^ 2
  RB_FMAC16("row_half_mirror", s2);       // lane ^ 7
  RB_FMAC16("row_ror:8", s3);             // lane ^ 8
  asm volatile("s_nop 1" ::);
  if constexpr (KEEP) {
    rb_stage_swap_keep<true>(v);
    rb_stage_swap_keep<false>(v);
  } else {
    ly_stage_swap<16, true>(v);
    ly_stage_swap<16, false>(v);
  }
}
#undef RB_FMAC16

template <bool IN_BF16>
__device__ __forceinline__ void rb_fetch(const void *in, size_t base, uint4 (&r)[IN_BF16 ? 2 : 4]) {
  if constexpr (IN_BF16) {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(in) + base;
    r[0] = *reinterpret_cast<const uint4 *>(p);
    r[1] = *reinterpret_cast<const uint4 *>(p + 512);
  } else {
    const float *p = reinterpret_cast<const float *>(in) + base;
    r[0] = *reinterpret_cast<const uint4 *>(p);
    r[1] = *reinterpret_cast<const uint4 *>(p + 4);
    r[2] = *reinterpret_cast<const uint4 *>(p + 512);
    r[3] = *reinterpret_cast<const uint4 *>(p + 516);
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void rb_unpack(const uint4 (&r)[IN_BF16 ? 2 : 4], float (&v)[16]) {
  if constexpr (IN_BF16) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w[4] = {r[h].x, r[h].y, r[h].z, r[h].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[8 * h + 2 * t] = __uint_as_float(w[t] << 16);
        v[8 * h + 2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[4 * q] = __uint_as_float(r[q].x);
      v[4 * q + 1] = __uint_as_float(r[q].y);
      v[4 * q + 2] = __uint_as_float(r[q].z);
      v[4 * q + 3] = __uint_as_float(r[q].w);
    }
  }
}

template <int NW, bool IN_BF16, bool OUT_BF16, bool TRANSPOSE>
__global__ void __launch_bounds__(1024)
rht_rows_blk(const void *in, void *out, int64_t rows, int n, int nb, const int8_t *signs, float *rowsum) {
  constexpr int E = 16, B = 64 * NW * E;
  using F = LyF<E, NW>;
  constexpr int logb = F::L + F::WB;
  static_assert((1 << logb) == B, "block size");
  extern __shared__ __attribute__((aligned(16))) float rb_buf[];   // nb (B + 64) floats when NW > 1
  __shared__ float red[16];
  const int tid = threadIdx.x;
  const int blk = tid / (64 * NW), tl = tid - blk * 64 * NW;
  float *buf = rb_buf + blk * (B + 64);
  const int eb = blk * B;
  const int el = 1024 * (tl >> 6) + 8 * rb_ell(tl & 63);   // element of register 0 (8.. at el + 512)
  const float inv = 1.0f / sqrtf((float)B);      // exact for even log2 B
  constexpr bool tr = NW > 1;                     // the labels are transposed iff the wave stages used LDS
  // sc: output scale, the sign after the transform or 1 / sqrt(B), times
  // rb_sgn of the label's lane. Input signs (applied before the transform):
  // float factors sg for float32 input; for bf16 input, the bf16 pairs
  // (s0, s1) and (s0, -s1) of the two elements of each packed word, so that
  // two dot products per word apply the signs and the first butterfly stage
  // (register stage 0 pairs exactly those two elements) with no unpacking
  // XO (bf16 in and out, one wave a block, B = 1024): the pairs carry
  // 1 / sqrt(B) = 2^-5 as well (an exact power of two: the sums are the same
  // values scaled), and sc reduces to a sign per element, applied to the
  // packed output words as sign-bit masks xm
  constexpr bool XO = IN_BF16 && OUT_BF16 && NW == 1;
  // one wave a block: the lane-swap stages keep their layout, and the
  // stores (and the output signs) follow rb_elem_out: register half h of
  // lane l is elements eo + 256 h .. + 7
  constexpr bool KEEP = NW == 1;
  const int eo = KEEP ? rb_elem_out(tl & 63, 0) : el;
  constexpr uint32_t ONE = XO ? (uint32_t)(127 - logb / 2) << 7 : 0x3F80u;   // bf16 2^-5 or 1
  float sg[IN_BF16 ? 1 : E], sc[E];
  uint32_t sp[IN_BF16 ? 8 : 1], sq[IN_BF16 ? 8 : 1], xm[XO ? 8 : 1];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = tr ? ly_elem<E, NW>(tl, i, true) : 16 * tl + i;
    const int pe = KEEP ? eo + (i & 7) + 256 * (i >> 3) : rb_elem(p);   // the element register i ends as
    sc[i] = rb_sgn((p >> 4) & 63) * (TRANSPOSE ? (float)signs[eb + pe] * inv : inv);
    const bool neg = !TRANSPOSE && signs[eb + el + (i & 7) + 512 * (i >> 3)] < 0;
    if constexpr (IN_BF16) {
      const uint32_t b = (neg ? 0x8000u : 0u) | ONE;   // bf16 -+1 (times 2^-5 under XO)
      if (i & 1) {
        sp[i >> 1] |= b << 16;
        sq[i >> 1] |= (b ^ 0x8000u) << 16;
      } else {
        sp[i >> 1] = b;
        sq[i >> 1] = b;
      }
    } else {
      sg[i] = neg ? -1.0f : 1.0f;
    }
    if constexpr (XO) {
      const uint32_t mb = sc[i] < 0.0f ? 0x8000u << (16 * (i & 1)) : 0u;
      xm[i >> 1] = (i & 1) ? xm[i >> 1] | mb : mb;
    }
  }
  uint4 raw[IN_BF16 ? 2 : 4];
  if ((int64_t)blockIdx.x < rows) rb_fetch<IN_BF16>(in, (size_t)blockIdx.x * n + eb + el, raw);
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const size_t base = (size_t)row * n + eb;
    float v[E];
    if constexpr (IN_BF16) {
      const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x2_t x2 = __builtin_bit_cast(bf16x2_t, w[j]);
        v[2 * j] = __builtin_amdgcn_fdot2_f32_bf16(x2, __builtin_bit_cast(bf16x2_t, sp[j]), 0.0f, false);
        v[2 * j + 1] = __builtin_amdgcn_fdot2_f32_bf16(x2, __builtin_bit_cast(bf16x2_t, sq[j]), 0.0f, false);
      }
    } else {
      rb_unpack<IN_BF16>(raw, v);
      if (!TRANSPOSE) {
#pragma unroll
        for (int i = 0; i < E; ++i) v[i] *= sg[i];
      }
    }
    if (row + gridDim.x < rows) rb_fetch<IN_BF16>(in, base + (size_t)gridDim.x * n + el, raw);   // next row
    rb_fwht_wave<IN_BF16 ? 1 : 0, KEEP>(v, tl & 63);
    if constexpr (NW > 1) {
      __syncthreads();                              // the previous row is out of buf
      ly_fwht_cross<E, NW>(v, buf, logb, tl);
    }
    float x[E];
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = XO ? v[i] : v[i] * sc[i];
    if constexpr (tr) {
      // back to the thread's own labels 16 tl + i through LDS, so that the
      // stores below are whole 16-byte vectors (the layout of ly_fwht_cross's
      // buffer: label p at p + 4 (p >> 10))
      __syncthreads();                              // every lane is done reading buf
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int p = ly_elem<E, NW>(tl, i, true);
        buf[p + 4 * (p >> 10)] = x[i];
      }
      __syncthreads();
      const float *r = buf + 16 * tl + 4 * (tl >> 6);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = reinterpret_cast<const float4 *>(r)[q];
        x[4 * q] = f.x; x[4 * q + 1] = f.y; x[4 * q + 2] = f.z; x[4 * q + 3] = f.w;
      }
    }
    float rs = 0.0f;
    if constexpr (OUT_BF16) {
      uint32_t w[E / 2];
#pragma unroll
      for (int i = 0; i < E; i += 2) {
        w[i / 2] = bf16x2_rne(x[i], x[i + 1]);
        if constexpr (XO) w[i / 2] ^= xm[i / 2];
      }
      if (rowsum) {
        // both halves of each packed word in one dot product with (1, 1)
        const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
        for (int i = 0; i < E / 2; ++i) rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), one, rs, false);
      }
      uint16_t *o = reinterpret_cast<uint16_t *>(out) + base + eo;
      *reinterpret_cast<uint4 *>(o) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4 *>(o + (KEEP ? 256 : 512)) = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      if (rowsum) {
#pragma unroll
        for (int i = 0; i < E; ++i) rs += x[i];
      }
      float *o = reinterpret_cast<float *>(out) + base + eo;
      constexpr int H1 = KEEP ? 256 : 512;
      reinterpret_cast<float4 *>(o)[0] = make_float4(x[0], x[1], x[2], x[3]);
      reinterpret_cast<float4 *>(o)[1] = make_float4(x[4], x[5], x[6], x[7]);
      reinterpret_cast<float4 *>(o + H1)[0] = make_float4(x[8], x[9], x[10], x[11]);
      reinterpret_cast<float4 *>(o + H1)[1] = make_float4(x[12], x[13], x[14], x[15]);
    }
    if (rowsum) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) rs += lane_xor(rs, off);
      if (NW == 1) __syncthreads();                 // (NW > 1: the barriers above) red is free
      if ((tid & 63) == 0) red[tid >> 6] = rs;
      __syncthreads();
      if (tid == 0) {
        float t = 0.0f;
        for (int w = 0; w < NW * nb; ++w) t += red[w];
        rowsum[row] = t;
      }
    }
  }
}

// ---------------------------------------------------------------- decode only
template <int BPW, bool OUT_F32>
__global__ void __launch_bounds__(256)
decode_weights_k(const uint16_t *idx1, const void *idx2, const uint8_t *blob, float scale,
                 const float *row_scale, uint32_t G, int64_t groups, void *out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  load_tables<BPW>(lds, blob);
  tables_landed();
  __syncthreads();
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t i1 = idx1[g];
    const uint32_t i2 = BPW == 2 ? 0u : load_idx2(idx2, g, BPW);
    const uint4 h = decode_group<BPW>(i1, i2, lds);
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    // the row's scale s_r = fl32(scale * row_scale[r]) (groups < 2^32)
    const float sr = row_scale ? scale * row_scale[(uint32_t)g / G] : scale;
    float w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = operand_value<BPW>((hw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
      w[t] = sr * v;                             // one float32 multiply
    }
    if constexpr (OUT_F32) {
      float4 *o = reinterpret_cast<float4 *>(out) + 2 * g;
      o[0] = make_float4(w[0], w[1], w[2], w[3]);
      o[1] = make_float4(w[4], w[5], w[6], w[7]);
    } else {
      uint32_t p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        p[t] = bf16x2_rne(w[2 * t], w[2 * t + 1]);
      reinterpret_cast<uint4 *>(out)[g] = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---------------------------------------------------------------- GEMV (m <= 16)
// Workgroup = 16 waves (4 per SIMD, so the SIMDs switch waves while loads are
// in flight), one 16-row weight tile n0 .. n0 + 15. The k axis is cut in
// chunks of 32 groups (256 inputs); wave w takes chunks w, w + 16, ... In a
// chunk, lane l (weight row j = l & 15, k-slot q = l >> 4) owns groups
// 32c + 8q .. 32c + 8q + 7 of row n0 + j (one 16-byte index load), and MFMA
// 16x16x32 step s contracts group 32c + 8q + s of every slot: A = x~ rows
// (m = l & 15, zero beyond m; the M side of the tile is the activation rows),
// B = decoded weights. All loads of a chunk are issued before its first
// decode. Partial sums of the 16 waves meet in LDS.
constexpr int GV_WAVES = 16;

// Index loads of 8 consecutive groups of one weight row, kept as loaded so
// that nothing waits for them until gv_unpack (a computation on a loaded
// value placed right after its load would stall the wave there).
struct GvRaw { uint4 a, b; };

template <int BPW, bool G8>
__device__ __forceinline__ GvRaw gv_load_raw(const uint16_t *idx1, const void *idx2, int64_t row, int64_t G,
                                             int64_t g0) {
  // row is clamped to the layer; groups past G are clamped (they meet zero weight operands)
  GvRaw r;
  if constexpr (G8) {
    const int64_t off = row * G + min(g0, G - 8);
    r.a = *reinterpret_cast<const uint4 *>(idx1 + off);
    if constexpr (BPW == 3) {
      const uint2 b = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(idx2) + off);
      r.b = make_uint4(b.x, b.y, 0u, 0u);
    } else if constexpr (BPW == 4) {
      r.b = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(idx2) + off);
    } else {
      r.b = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    uint32_t w1[8], w2[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t o = row * G + min(g0 + u, G - 1);
      w1[u] = idx1[o];
      w2[u] = BPW == 2 ? 0u : load_idx2(idx2, o, BPW);
    }
    r.a = make_uint4(w1[0] | (w1[1] << 16), w1[2] | (w1[3] << 16), w1[4] | (w1[5] << 16), w1[6] | (w1[7] << 16));
    if constexpr (BPW == 3)
      r.b = make_uint4(w2[0] | (w2[1] << 8) | (w2[2] << 16) | (w2[3] << 24),
                       w2[4] | (w2[5] << 8) | (w2[6] << 16) | (w2[7] << 24), 0u, 0u);
    else
      r.b = make_uint4(w2[0] | (w2[1] << 16), w2[2] | (w2[3] << 16), w2[4] | (w2[5] << 16), w2[6] | (w2[7] << 16));
  }
  return r;
}

// i1 = i' = i - 1 mod 2^16 of stage 1; i2 = i' of stage 2 at 4 bpw, the plain
// residual row at 3 bpw
template <int BPW>
__device__ __forceinline__ void gv_unpack(const GvRaw &r, uint32_t (&i1)[8], uint32_t (&i2)[8]) {
  const uint32_t w[4] = {pk_dec16(r.a.x), pk_dec16(r.a.y), pk_dec16(r.a.z), pk_dec16(r.a.w)};
#pragma unroll
  for (int u = 0; u < 4; ++u) { i1[2 * u] = w[u] & 0xFFFFu; i1[2 * u + 1] = w[u] >> 16; }
  if constexpr (BPW == 3) {
#pragma unroll
    for (int u = 0; u < 4; ++u) { i2[u] = (r.b.x >> (8 * u)) & 0xFFu; i2[4 + u] = (r.b.y >> (8 * u)) & 0xFFu; }
  } else if constexpr (BPW == 4) {
    const uint32_t x[4] = {pk_dec16(r.b.x), pk_dec16(r.b.y), pk_dec16(r.b.z), pk_dec16(r.b.w)};
#pragma unroll
    for (int u = 0; u < 4; ++u) { i2[2 * u] = x[u] & 0xFFFFu; i2[2 * u + 1] = x[u] >> 16; }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) i2[u] = 0u;
  }
}

// TILED: x~ in the operand layout of tile16_index (k a multiple of 256), so
// that each operand load is one contiguous KiB; otherwise x~ row-major [m][k].
template <int BPW, bool G8, int RT, bool TILED>
__global__ void __launch_bounds__(64 * GV_WAVES, 1)
gemv_bf16(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const uint16_t *xt,
          const float *rowsum, int64_t m, int64_t n, int64_t k, float post, const float *row_scale,
          void *out, glq_dtype out_dt) {
  // RT tiles of 16 weight rows per workgroup share every x~ operand load
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + lds_table_bytes<BPW>());   // [RT][waves][16][16]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * RT;
  const int64_t G = k / 8;
  const int64_t chunks = (G + 31) / 32;
  const uint16_t *xrow = xt + (size_t)min((int64_t)j, m - 1) * k;

  // The first chunk's loads go out before the table copy; later chunks (k >
  // 4096) are loaded one at a time: the other waves of the SIMD hide the wait.
  // All loads are unconditional with clamped addresses (a select on a loaded
  // value would make each load a branch that waits for it): x~ rows past m
  // only feed output rows that are not stored, and groups past k meet zero
  // weight operands.
  int64_t c = wave;
  GvRaw raw[RT];
  uint4 av[8];
  auto load_chunk = [&](int64_t cc) {
    const int64_t g0 = 32 * cc + 8 * q;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) raw[rt] = gv_load_raw<BPW, G8>(idx1, idx2, min(n0 + 16 * rt + j, n - 1), G, g0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if constexpr (TILED) av[s] = *reinterpret_cast<const uint4 *>(xt + ((size_t)((cc * 8 + s) * 64 + lane) << 3));
      else av[s] = *reinterpret_cast<const uint4 *>(xrow + 8 * min(g0 + s, G - 1));
    }
  };
  if (c < chunks) load_chunk(c);
  // row sum of the activation row this thread reduces at the end (loaded
  // unconditionally, clamped, used only after the reduction)
  float rs_raw = 0.0f;
  if constexpr (Epi<BPW>::bias != 0.0f) rs_raw = rowsum[min((int64_t)((threadIdx.x >> 4) & 15), m - 1)];
  load_tables<BPW, 64 * GV_WAVES>(lds, blob);
  tables_landed();
  __syncthreads();
  f32x4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  while (c < chunks) {
    const int64_t g0 = 32 * c + 8 * q;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t i1[8], i2[8];
      gv_unpack<BPW>(raw[rt], i1, i2);
      Dec8<BPW> D;
      uint4 bv[8];
      D.run(i1, i2, bv);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 b = g0 + s < G ? bv[s] : make_uint4(0, 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[s]),
                                                          __builtin_bit_cast(bf16x8, b), acc[rt], 0, 0, 0);
      }
    }
    c += GV_WAVES;
    if (c < chunks) load_chunk(c);
  }
  // D[r][col]: lane holds rows 4 (lane >> 4) + t (activation row), column lane & 15 (weight row)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[((rt * GV_WAVES + wave) * 16 + 4 * q + t) * 16 + j] = acc[rt][t];
  __syncthreads();
  if (threadIdx.x < 256 * RT) {
    const int rt = threadIdx.x >> 8, r = (threadIdx.x >> 4) & 15, col = threadIdx.x & 15;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < GV_WAVES; ++w) v += red[((rt * GV_WAVES + w) * 16 + r) * 16 + col];
    const int64_t nrow = n0 + 16 * rt + col;
    if (r < m && nrow < n) {
      const float pr = row_scale ? post * row_scale[nrow] : post;
      store_out(out, out_dt, (size_t)r * n + nrow, pr * (v - Epi<BPW>::bias * rs_raw));
    }
  }
}

// ---------------------------------------------------------------- whole layer (m <= 4)
// One launch for y = U^T (s W^) (V x) at a few activation rows (decode-time
// batch sizes), where separate RHT launches would cost more than the
// decode-GEMV itself. Every workgroup: issues its x and input-sign loads, then
// its first index loads and the table copy, rotates x while the tables are
// in flight (block FWHT along k in registers and lane exchanges, one LDS
// transpose, 1/sqrt(b), bf16 rounding, row sums at 3 and 4 bpw), runs the
// 16-wave decode-GEMV of gemv_bf16 over its 16-row weight tiles with the x~
// operands read from LDS, and writes z (float32) to the workspace with
// write-through stores. Tickets on 16 group counters and one top counter
// (each reset by its last taker) pick the last workgroup, which loads all of
// z and the output signs, applies U^T (block FWHT along n, then signs) and
// writes y.
constexpr int LY_MAXE = 16384;                       // m*k and m*n limit (64 KiB of float32)
constexpr int LY_THREADS = 64 * GV_WAVES;            // 1024
// float32 transpose buffer (padded); it also holds x~ in bf16 and, past
// x~, the cross-wave reduction rows and the row sums (see layer_small)
constexpr size_t LY_BUF_BYTES = (LY_MAXE + 4 * 16) * 4 + 64;

// The table image rounded up to whole 1 KiB copy runs (the tail of the last
// run lands in padding that nothing reads).
template <int BPW>
constexpr uint32_t ly_tab_bytes() { return (lds_table_bytes<BPW>() + 1023) / 1024 * 1024; }

template <int BPW>
constexpr size_t ly_lds_bytes() { return ly_tab_bytes<BPW>() + LY_BUF_BYTES; }
static_assert(ly_lds_bytes<3>() <= 160 * 1024, "single-launch layer fits the LDS of a CU");

// Table copy of the single-launch layer, staged through registers: global
// loads that the rotation of x, issued after the x loads, does not wait for
// (a copy straight to LDS counts as a different kind of load, after which the
// compiler waits for all loads at the first use of any), written to LDS once
// x~ is done. Every wave copies the same fixed number of 1 KiB runs with no
// branch; lanes past the image read clamped blob addresses and write the
// padding, and waves past the last run repeat it (the same bytes to the same
// place). Workgroups start at different runs (rot), so that the 32 workgroups
// of an XCD do not all ask the same L2 channel for the same lines at once.
template <int BPW> struct LyTab {   // named members: an array here ended up on the stack
  static constexpr uint32_t runs = ly_tab_bytes<BPW>() / 1024, per_wave = (runs + GV_WAVES - 1) / GV_WAVES;
  static_assert(per_wave <= 6, "table runs per wave");
  uint4 v0, v1, v2, v3, v4, v5;
};

template <int BPW>
__device__ __forceinline__ uint32_t ly_run(uint32_t u, uint32_t rot) {
  constexpr uint32_t runs = LyTab<BPW>::runs;
  const uint32_t r = min((uint32_t)(threadIdx.x >> 6) + GV_WAVES * u, runs - 1) + rot;   // rot < runs
  return r >= runs ? r - runs : r;
}

template <int BPW>
__device__ __forceinline__ uint4 ly_fetch_run(const uint8_t *blob, uint32_t u, uint32_t rot) {
  const uint32_t pos = 1024 * ly_run<BPW>(u, rot) + 16 * (threadIdx.x & 63);
  return *reinterpret_cast<const uint4 *>(blob + min(table_src<BPW>(pos), kBlobBytes - 16));
}

template <int BPW>
__device__ __forceinline__ void ly_fetch_tables(const uint8_t *blob, uint32_t rot, LyTab<BPW> &t) {
  constexpr uint32_t pw = LyTab<BPW>::per_wave;
  t.v0 = ly_fetch_run<BPW>(blob, 0, rot);
  if constexpr (pw > 1) t.v1 = ly_fetch_run<BPW>(blob, 1, rot);
  if constexpr (pw > 2) t.v2 = ly_fetch_run<BPW>(blob, 2, rot);
  if constexpr (pw > 3) t.v3 = ly_fetch_run<BPW>(blob, 3, rot);
  if constexpr (pw > 4) t.v4 = ly_fetch_run<BPW>(blob, 4, rot);
  if constexpr (pw > 5) t.v5 = ly_fetch_run<BPW>(blob, 5, rot);
}

template <int BPW>
__device__ __forceinline__ void ly_store_tables(uint8_t *lds, uint32_t rot, const LyTab<BPW> &t) {
  constexpr uint32_t pw = LyTab<BPW>::per_wave;
  const uint32_t l16 = 16 * (threadIdx.x & 63);
  *reinterpret_cast<uint4 *>(lds + 1024 * ly_run<BPW>(0, rot) + l16) = t.v0;
  if constexpr (pw > 1) *reinterpret_cast<uint4 *>(lds + 1024 * ly_run<BPW>(1, rot) + l16) = t.v1;
  if constexpr (pw > 2) *reinterpret_cast<uint4 *>(lds + 1024 * ly_run<BPW>(2, rot) + l16) = t.v2;
  if constexpr (pw > 3) *reinterpret_cast<uint4 *>(lds + 1024 * ly_run<BPW>(3, rot) + l16) = t.v3;
  if constexpr (pw > 4) *reinterpret_cast<uint4 *>(lds + 1024 * ly_run<BPW>(4, rot) + l16) = t.v4;
  if constexpr (pw > 5) *reinterpret_cast<uint4 *>(lds + 1024 * ly_run<BPW>(5, rot) + l16) = t.v5;
}

// Control words of the single-launch layer at the start of the workspace:
// group counters g = 0 .. 15 at byte 256 g, the top counter at byte 4096 (each
// on its own cache line, so the tickets of different groups do not contend).
constexpr int LY_GROUPS = 16;
constexpr size_t kCtrlBytes = GLQ_WS_CTRL_BYTES;
static_assert(kCtrlBytes % 256 == 0 && kCtrlBytes >= 4096 + 4, "ticket counters fit");

// Input side. Issue order: this thread's x and input-sign loads, the first
// index loads of the decode (raw), the table loads; then x~ = bf16( H (sign_k
// . x) / sqrt(b) ) into xb (LDS, [m][k] bf16), which waits for the x loads
// only, and (ROWSUM) per-wave row-sum partials into red[wave * 4 + r]. Ends
// with this wave's table runs written to LDS and the barrier that publishes
// tables, xb and red. Loads use clamped in-bounds addresses; elements past m k are zeroed
// and, being whole Hadamard blocks of their own, never reach a stored value.
// xb lies past the transpose buffer for E <= 8 and on top of it for E = 16.
template <int BPW, int E, bool ROWSUM, bool FULL>
__device__ __forceinline__ void ly_input(const uint16_t *x, const int8_t *sign_k, int mk, int k, int logbk,
                                         uint8_t *lds, float *buf, uint16_t *xb, float *red, int tid, const uint16_t *idx1,
                                         const void *idx2, const uint8_t *blob, uint32_t rot, int64_t irow,
                                         int64_t G, int64_t ig0, GvRaw &raw) {
  const int e0 = E * tid, el = min(e0, mk - E);      // mk % E == 0
  uint32_t xw[(E + 1) / 2], sw[(E + 3) / 4];
  if constexpr (E == 1) { xw[0] = x[el]; sw[0] = (uint8_t)sign_k[el % k]; }
  else if constexpr (E == 2) {
    xw[0] = *reinterpret_cast<const uint32_t *>(x + el);
    sw[0] = *reinterpret_cast<const uint16_t *>(sign_k + el % k);
  } else if constexpr (E == 4) {
    const uint2 u = *reinterpret_cast<const uint2 *>(x + el);
    xw[0] = u.x; xw[1] = u.y;
    sw[0] = *reinterpret_cast<const uint32_t *>(sign_k + el % k);
  } else {
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      const uint4 u = *reinterpret_cast<const uint4 *>(x + el + 8 * c);
      xw[4 * c] = u.x; xw[4 * c + 1] = u.y; xw[4 * c + 2] = u.z; xw[4 * c + 3] = u.w;
      const uint2 g = *reinterpret_cast<const uint2 *>(sign_k + (el + 8 * c) % k);
      sw[2 * c] = g.x; sw[2 * c + 1] = g.y;
    }
  }
  raw = gv_load_raw<BPW, true>(idx1, idx2, irow, G, ig0);
  LyTab<BPW> tab;
  ly_fetch_tables<BPW>(blob, rot, tab);
  __builtin_amdgcn_sched_barrier(0);                 // everything above is issued before the first wait
  const float keep = FULL || e0 < mk ? 1.0f : 0.0f;    // FULL: m k = 1024 E
  float v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float sg = (float)(int8_t)((sw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    const float xv = __uint_as_float(((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16);
    v[i] = FULL ? xv * sg : xv * (sg * keep);
  }
  const bool tr = ly_fwht<E, 16, FULL>(v, buf, logbk, tid);
  const float inv = 1.0f / sqrtf((float)(1 << logbk));
  uint16_t h[E];
#pragma unroll
  for (int i = 0; i < E; i += 2) {
    const uint32_t hh = bf16x2_rne(v[i] * inv, i + 1 < E ? v[i + 1] * inv : 0.0f);
    h[i] = (uint16_t)hh;
    if (i + 1 < E) h[i + 1] = (uint16_t)(hh >> 16);
  }
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (ROWSUM) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int e = ly_elem<E>(tid, i, tr);
      if (e < mk) {
        const float hv = __uint_as_float((uint32_t)h[i] << 16);
        const int r = (e >= k) + (e >= 2 * k) + (e >= 3 * k);   // m <= 4
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) rs[rr] += rr == r ? hv : 0.0f;
      }
    }
  }
  if (E == 16 && tr) __syncthreads();                // every thread has read buf (xb aliases it)
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = ly_elem<E>(tid, i, tr);
    if (e < mk) xb[e] = h[i];
  }
  if constexpr (ROWSUM) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if (rr * k >= mk) break;                        // rows past m
      float t = rs[rr];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) t += lane_xor(t, off);
      if ((tid & 63) == 0) red[(tid >> 6) * 4 + rr] = t;
    }
  }
  ly_store_tables<BPW>(lds, rot, tab);
  __syncthreads();
}

// Output side (last workgroup): y = sign_n . H z / sqrt(b). The signs this
// thread applies (to elements ly_elem(tid, i, logbn > L)) are loaded after z,
// so that the first butterflies wait for z alone.
template <int E, bool FULL>
__device__ __forceinline__ void ly_output(const float *z, const int8_t *sign_n, int n, int mn, int logbn,
                                          float *buf, void *y, glq_dtype y_dt, int tid) {
  float v[E];
  const int e0 = E * tid;
#pragma unroll
  for (int i = 0; i < E; ++i)   // padding elements form whole blocks of their own
    v[i] = e0 + i < mn ? __hip_atomic_load(z + e0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
  int sn[E];
  {
    const bool str = logbn > LyF<E>::L;
#pragma unroll
    for (int i = 0; i < E; ++i) sn[i] = sign_n[min(ly_elem<E>(tid, i, str), mn - 1) % n];
  }
  const bool tr = ly_fwht<E, 16, FULL>(v, buf, logbn, tid);
  const float inv = 1.0f / sqrtf((float)(1 << logbn));
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = ly_elem<E>(tid, i, tr);
    if (e < mn) store_out(y, y_dt, (size_t)e, v[i] * inv * (float)(int8_t)sn[i]);
  }
}

// Output side for one row of n = 1024 NW (the Hadamard block is all of n):
// waves 0 .. NW - 1 hold 16 elements a lane, lane l of wave w the elements
// 1024 w + 256 j + 4 rb_ell(l) + 0..3 (j = 0..3, registers 4 j ..), so that z
// comes in as four 16-byte coherent loads a lane, each covering one
// contiguous KiB of the wave (per-element loads fetched every line 16 times),
// and y goes out in 8- or 16-byte stores. The FWHT over a wave's 1024
// elements is rb_fwht_wave (register bits are element bits 0, 1, 8, 9, the
// relabelled lane bits element bits 2..7), the bits above the wave one LDS
// transpose (ly_fwht_cross) and one back. Every thread of the workgroup
// takes part in the barriers.
__device__ __forceinline__ int lo_elem(int p) {
  return (p & ~1023) | (p & 3) | (((p >> 2) & 3) << 8) | (rb_ell((p >> 4) & 63) << 2);
}

template <int NW>
__device__ __forceinline__ void ly_output_rb(const float *z, const int8_t *sign_n, int n, float *buf, void *y,
                                             glq_dtype y_dt, int tid) {
  constexpr int B = 1024 * NW;
  const bool act = tid < 64 * NW;                    // whole waves
  const int lane = tid & 63;
  const int el = 1024 * (tid >> 6) + 4 * rb_ell(lane);   // element of register 0 (4 j + t at el + 256 j + t)
  float v[16];
  if (act) {
    // coherent (sc1) loads, as the relaxed agent-scope loads of z elsewhere
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)z, 0, 4 * B, 0x00020000);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (el + 256 * j), 0, 16));
      v[4 * j] = __uint_as_float(u.x); v[4 * j + 1] = __uint_as_float(u.y);
      v[4 * j + 2] = __uint_as_float(u.z); v[4 * j + 3] = __uint_as_float(u.w);
    }
    rb_fwht_wave(v, lane);
  }
  const float inv = 1.0f / sqrtf((float)B);
  if constexpr (NW > 1) {
    // the bits above the wave, then back to the thread's own labels 16 tid + i
    if (act) {
      float *w = buf + 16 * tid + 4 * (tid >> 6);
#pragma unroll
      for (int i = 0; i < 16; i += 4) *reinterpret_cast<float4 *>(w + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    }
    __syncthreads();
    if (act) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hi = i % NW;
        v[i] = buf[tid + 64 * NW * (i / NW) + (hi << 10) + 4 * hi];
      }
#pragma unroll
      for (int h = 0; h < LyF<16, NW>::WB; ++h) ly_stage_regs<16>(v, h);
    }
    __syncthreads();                                 // every lane is done reading buf
    if (act) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = ly_elem<16, NW>(tid, i, true);
        buf[p + 4 * (p >> 10)] = v[i] * (inv * rb_sgn((p >> 4) & 63));
      }
    }
    __syncthreads();
    if (act) {
      const float *r = buf + 16 * tid + 4 * (tid >> 6);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = reinterpret_cast<const float4 *>(r)[q];
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
    }
  } else {
    const float c = inv * rb_sgn(lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= c;
  }
  if (!act) return;
  // labels 16 tid + i are elements el + 256 j + t (i = 4 j + t): signs, store
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = el + 256 * j;
    const uint32_t sw = *reinterpret_cast<const uint32_t *>(sign_n + e);
    float o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = v[4 * j + t] * (float)(int8_t)((sw >> (8 * t)) & 0xFFu);
    if (y_dt == GLQ_BF16)
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + e) = make_uint2(bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3]));
    else
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + e) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

template <int BPW>
__global__ void __launch_bounds__(LY_THREADS, 1)
layer_small(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const uint16_t *x,
            const int8_t *sign_k, const int8_t *sign_n, int64_t m, int64_t n, int64_t k, int logbk,
            int logbn, float post, const float *row_scale, void *y, glq_dtype y_dt, float *z,
            unsigned int *ctrl) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *xs = reinterpret_cast<float *>(lds + ly_tab_bytes<BPW>());
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int64_t G = k / 8, chunks = (G + 31) / 32;
  const int64_t tiles = (n + 15) / 16;               // >= gridDim.x
  const int mk = (int)(m * k), mn = (int)(m * n);
  const int ei = ly_e(mk);
  // x~ as bf16 [m][k] after rotation: past the transpose buffer's 1024 E + 64
  // floats when E <= 8, on top of it at E = 16. The reduction rows (16 waves
  // x 256 floats) and misc follow x~ at its largest (2048 E bytes), or the
  // upper half of the buffer at E = 16 (free once x~ is written): they are
  // written only after the last read of the transpose buffer in the input
  // transform, and the output transform reuses the buffer only after the
  // last workgroup has read its flag.
  uint16_t *xb = reinterpret_cast<uint16_t *>(ei <= 8 ? xs + 1024 * ei + 64 : xs);
  float *red = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(xs) +
                                         (ei == 16 ? 32768 : (1024 * ei + 64) * 4 + 2048 * ei));
  float *misc = red + GV_WAVES * 256;                 // [0..3] row sums, [8] last-workgroup flag

  // 1. x, the first index loads and the table copy; x~ into LDS while the
  // tables land (the barrier at its end publishes tables, x~ and row sums)
  int64_t tile = blockIdx.x, c = wave;
  GvRaw raw;
  {
    constexpr bool RS = Epi<BPW>::bias != 0.0f;
    const uint32_t rot = (blockIdx.x >> 3) % (ly_tab_bytes<BPW>() / 1024);
    const int64_t irow = min(tile * 16 + j, n - 1), ig0 = 32 * min(c, chunks - 1) + 8 * q;
#define GLQ_LY_IN(E, F) ly_input<BPW, E, RS, F>(x, sign_k, mk, (int)k, logbk, lds, xs, xb, red, tid, idx1, idx2, \
                                              blob, rot, irow, G, ig0, raw)
    // FULL variants for one row whose block is all of k (k = 4096, 8192, 16384)
    switch (ei) {
      case 1: GLQ_LY_IN(1, false); break;
      case 2: GLQ_LY_IN(2, false); break;
      case 4: if (logbk == LyF<4>::L + 4) GLQ_LY_IN(4, true); else GLQ_LY_IN(4, false); break;
      case 8: if (logbk == LyF<8>::L + 4) GLQ_LY_IN(8, true); else GLQ_LY_IN(8, false); break;
      default: if (logbk == LyF<16>::L + 4) GLQ_LY_IN(16, true); else GLQ_LY_IN(16, false); break;
    }
#undef GLQ_LY_IN
    if (RS && tid < m) {
      float t = 0.0f;
      for (int w = 0; w < GV_WAVES; ++w) t += red[w * 4 + tid];
      misc[tid] = t;                                 // read after the next barrier
    }
  }
  // 3. decode-GEMV over this workgroup's tiles
  const uint16_t *xrow = xb + (size_t)min((int64_t)j, m - 1) * k;
  for (; tile < tiles; tile += gridDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (c = wave; c < chunks; c += GV_WAVES) {
      // the indices of this wave's next chunk (this tile's, else the next
      // tile's first) are in flight while this one decodes; past the last
      // chunk the clamped addresses load indices that are never used
      const bool wrap = c + GV_WAVES >= chunks;
      const int64_t cn = wrap ? wave : c + GV_WAVES, tn = wrap ? tile + gridDim.x : tile;
      const GvRaw rawn = gv_load_raw<BPW, true>(idx1, idx2, min(tn * 16 + j, n - 1), G,
                                                32 * min(cn, chunks - 1) + 8 * q);
      const int64_t g0 = 32 * c + 8 * q;
      uint32_t i1[8], i2[8];
      gv_unpack<BPW>(raw, i1, i2);
      Dec8<BPW> D;
      uint4 bv[8];
      D.run(i1, i2, bv);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        // x~ rows past m feed output rows that are not stored; groups past k
        // meet zero weight operands
        const uint4 av = *reinterpret_cast<const uint4 *>(xrow + 8 * min(g0 + s, G - 1));
        const uint4 b = g0 + s < G ? bv[s] : make_uint4(0, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
      }
      raw = rawn;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) red[(wave * 16 + 4 * q + t) * 16 + j] = acc[t];
    __syncthreads();
    if (tid < 256) {
      const int r = tid >> 4, col = tid & 15;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < GV_WAVES; ++w) v += red[(w * 16 + r) * 16 + col];
      const int64_t nrow = tile * 16 + col;
      if (r < m && nrow < n) {
        if (Epi<BPW>::bias != 0.0f) v -= Epi<BPW>::bias * misc[r];
        const float pr = row_scale ? post * row_scale[nrow] : post;
        // coherent (write-through) store: visible to every XCD without an L2 writeback
        __hip_atomic_store(z + (size_t)r * n + nrow, pr * v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
  // 4. tickets. z went out with coherent stores; once they have completed
  // (s_waitcnt) the workgroup takes a ticket of its group counter; the last
  // taker of each group takes one of the top counter, and the last taker of
  // that one applies U^T. (A threadfence here would write back the whole L2
  // of the XCD, once per workgroup.)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned int g = blockIdx.x % LY_GROUPS;
    const unsigned int ngroups = min(gridDim.x, (unsigned)LY_GROUPS);
    const unsigned int in_group = (gridDim.x - g + LY_GROUPS - 1) / LY_GROUPS;   // workgroups b with b % 16 == g
    unsigned int *gc = ctrl + 64 * g, *top = ctrl + 1024;
    float last = 0.0f;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == in_group - 1) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = 1.0f;
      }
    }
    misc[8] = last;
  }
  __syncthreads();
  if (misc[8] == 0.0f) return;
  __syncthreads();                                   // every thread has read the flag (the buffer below overlaps it)
  // 5. the last workgroup: y = U^T z
#define GLQ_LY_OUT(E, F) ly_output<E, F>(z, sign_n, (int)n, mn, logbn, xs, y, y_dt, tid)
  // one row whose Hadamard block is all of n = 8192 or 16384, aligned y and
  // signs: 16-byte coherent loads of z, vector stores of y (16384: the tail
  // 10.4 -> 4.2 us; at n = 4096 the 16-wave path below measured level)
  const bool rb = m == 1 && n >= 8192 && (1 << logbn) == n &&
                  ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(sign_n)) & 15) == 0;
  if (rb) {
    switch (n >> 10) {
      case 1: ly_output_rb<1>(z, sign_n, (int)n, xs, y, y_dt, tid); return;
      case 2: ly_output_rb<2>(z, sign_n, (int)n, xs, y, y_dt, tid); return;
      case 4: ly_output_rb<4>(z, sign_n, (int)n, xs, y, y_dt, tid); return;
      case 8: ly_output_rb<8>(z, sign_n, (int)n, xs, y, y_dt, tid); return;
      default: ly_output_rb<16>(z, sign_n, (int)n, xs, y, y_dt, tid); return;
    }
  }
  switch (ly_e(mn)) {
    case 1: GLQ_LY_OUT(1, false); break;
    case 2: GLQ_LY_OUT(2, false); break;
    case 4: if (logbn == LyF<4>::L + 4) GLQ_LY_OUT(4, true); else GLQ_LY_OUT(4, false); break;
    case 8: if (logbn == LyF<8>::L + 4) GLQ_LY_OUT(8, true); else GLQ_LY_OUT(8, false); break;
    default: if (logbn == LyF<16>::L + 4) GLQ_LY_OUT(16, true); else GLQ_LY_OUT(16, false); break;
  }
#undef GLQ_LY_OUT
}

// ---------------------------------------------------------------- GEMM (m > 16)
// Workgroup tile 256 (activation rows) x 256 (weight rows), 4 waves; wave w
// owns weight rows n0 + 64w .. +63 for all 256 activation rows: 8 x 2 tiles of
// MFMA 32x32x16 (bf16) whose B operands it decodes itself, straight into
// registers (no weight tile goes through LDS). A k-step covers 64 inputs =
// 8 groups; MFMA sub-step u (0..3) contracts, in k-slot p = lane >> 5,
// group 8s + 4p + u, so lane (c = lane & 31, p) needs groups 8s + 4p .. +3 of
// weight rows n0 + 32t + c: one 8-byte index load per tile. x~ is staged
// through a double-buffered LDS tile [256][64 + 8] (one barrier per k-step),
// fetched from global memory one step ahead into registers.
//   MFMA 32x32x16 operand layout: A lane l = row l & 31, k 8(l >> 5) .. +7;
//   B lane l = column l & 31, k 8(l >> 5) .. +7; D register i of lane l =
//   row 8(i >> 2) + 4(l >> 5) + (i & 3), column l & 31.
constexpr int GM_BM = 256, GM_BN = 256, GM_BK = 64, GM_LDA = GM_BK + 8;
constexpr size_t GM_A_BYTES = (size_t)GM_BM * GM_LDA * 2;   // one buffer

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Index planes for k-step s: rows nrow0 + 32 t + c (t = 0, 1), groups
// 8 s + 4 p .. +3, returned as stored (gm_dec_idx turns them into
// i' = i - 1 mod 2^16 where they are used, so nothing waits for the loads
// early). Addresses are clamped into the planes instead of branching:
// out-of-range rows are never stored, out-of-range groups meet zero
// activations, and any index decodes to finite values. G4: k/8 is a
// multiple of 4, so the 4 indices are one aligned 8-byte load.
template <int BPW, bool G4>
__device__ __forceinline__ void gm_load_idx(const uint16_t *idx1, const void *idx2, int64_t n,
                                            int64_t G, int64_t nrow0, int c, int p, int64_t s,
                                            uint2 (&i1)[2], uint2 (&i2)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t row = min(nrow0 + 32 * t + c, n - 1);
    if constexpr (G4) {
      const int64_t off = row * G + min(8 * s + 4 * p, G - 4);
      i1[t] = *reinterpret_cast<const uint2 *>(idx1 + off);
      if constexpr (BPW == 3) i2[t] = make_uint2(*reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(idx2) + off), 0u);
      if constexpr (BPW == 4) i2[t] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(idx2) + off);
      if constexpr (BPW == 2) i2[t] = make_uint2(0u, 0u);
    } else {
      uint32_t w1[4], w2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t o = row * G + min(8 * s + 4 * p + u, G - 1);
        w1[u] = idx1[o];
        w2[u] = BPW > 2 ? load_idx2(idx2, o, BPW) : 0u;
      }
      i1[t] = make_uint2(w1[0] | (w1[1] << 16), w1[2] | (w1[3] << 16));
      if constexpr (BPW == 3) i2[t] = make_uint2(w2[0] | (w2[1] << 8) | (w2[2] << 16) | (w2[3] << 24), 0u);
      else i2[t] = make_uint2(w2[0] | (w2[1] << 16), w2[2] | (w2[3] << 16));
    }
  }
}

// stored indices -> i' = i - 1 mod 2^16 (stage 1; stage 2 at 4 bpw)
template <int BPW>
__device__ __forceinline__ void gm_dec_idx(uint2 (&i1)[2], uint2 (&i2)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    i1[t] = make_uint2(pk_dec16(i1[t].x), pk_dec16(i1[t].y));
    if constexpr (BPW == 4) i2[t] = make_uint2(pk_dec16(i2[t].x), pk_dec16(i2[t].y));
  }
}

// x~ tile of k-step s: 256 rows x 64 inputs (128 B per row); piece
// pc = tid + 256 u is row pc >> 3, 16-byte column pc & 7. The loads are
// unconditional with clamped addresses: rows past m only feed accumulator rows
// that are never stored, and columns past k are zeroed when the tile is
// written to LDS (a select on the loaded value here would turn the loads into
// branches and make the wave wait for them at once).
__device__ __forceinline__ void gm_load_a(const uint16_t *xt, int64_t m, int64_t k, int64_t m0, int64_t s,
                                          uint4 (&ra)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pc = threadIdx.x + 256 * u;
    const int64_t r = min(m0 + (pc >> 3), m - 1);
    const int64_t kk = min(GM_BK * s + 8 * (pc & 7), k - 8);
    ra[u] = *reinterpret_cast<const uint4 *>(xt + (size_t)r * k + kk);
  }
}

// kvalid = inputs of this tile that lie inside [0, k) (uniform)
__device__ __forceinline__ void gm_store_a(uint16_t *As, const uint4 (&ra)[8], int64_t kvalid) {
  if (kvalid >= GM_BK) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pc = threadIdx.x + 256 * u;
      *reinterpret_cast<uint4 *>(As + (pc >> 3) * GM_LDA + 8 * (pc & 7)) = ra[u];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pc = threadIdx.x + 256 * u;
      const bool ok = 8 * (pc & 7) < kvalid;
      *reinterpret_cast<uint4 *>(As + (pc >> 3) * GM_LDA + 8 * (pc & 7)) = ok ? ra[u] : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int BPW>
__device__ __forceinline__ uint4 gm_decode_one(const uint2 (&i1)[2], const uint2 (&i2)[2], int t, int u,
                                               const uint8_t *lds) {
  const uint32_t w1 = u < 2 ? i1[t].x : i1[t].y;
  const uint32_t a1 = (w1 >> (16 * (u & 1))) & 0xFFFFu;
  uint32_t a2 = 0;
  if constexpr (BPW == 3) a2 = (i2[t].x >> (8 * u)) & 0xFFu;
  if constexpr (BPW == 4) a2 = ((u < 2 ? i2[t].x : i2[t].y) >> (16 * (u & 1))) & 0xFFFFu;
  (void)lds;
  return decode_ip<BPW>(a1, a2);
}

// GEMM epilogue: z = post * acc + cz(row) with cz = -post * bias * rowsum(x~),
// staged through LDS (free once the k-loop has ended) so that every lane
// stores 16 contiguous bytes of an output row. Each wave stages its own
// 32 MB x 32 NT tile in chunks of CH 32-row blocks. vec: 16-byte stores are
// aligned (n * element size % 16 == 0 and an aligned output pointer).
template <int BPW, bool OUT_BF16, int NT = 2, int MB = 8>
__device__ __forceinline__ void gm_epilogue(const f32x16 (&acc)[MB][NT], const float *rowsum, float post,
                                            const float *row_scale, void *out, int64_t m, int64_t n, int64_t m0,
                                            int64_t n0, int lane, int wave, bool vec) {
  constexpr int ES = OUT_BF16 ? 2 : 4;              // bytes per output value
  constexpr int CH = OUT_BF16 ? 4 : 2;              // 32-row blocks per chunk
  constexpr uint32_t SB = 32 * NT * ES + 16;        // padded LDS row stride (bytes)
  constexpr uint32_t WAVE_BYTES = 32 * CH * SB;
  constexpr int CPR = 32 * NT * ES / 16;            // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;                     // rows per pass of the wave
  constexpr int EPP = 16 / ES;                      // values per piece
  const int c = lane & 31, p = lane >> 5;
  const uint32_t wbase = wave * WAVE_BYTES;
  const int64_t rlast4 = ((m - 1) >> 2) << 2;
  // per output column (weight row) n0 + 32 t + c: post, times its row scale
  float pt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) pt[t] = row_scale ? post * row_scale[min(n0 + 32 * t + c, n - 1)] : post;
#pragma unroll
  for (int a0 = 0; a0 < MB; a0 += CH) {
#pragma unroll
    for (int a = a0; a < a0 + CH; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float cz[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (Epi<BPW>::bias != 0.0f) {
          // rows r0 .. r0 + 3 (r0 % 4 == 0); the clamped 16-byte load stays
          // inside the 256-byte-aligned row-sum buffer
          const int64_t r0 = min(m0 + 32 * a + 8 * q + 4 * p, rlast4);
          const float4 rs = *reinterpret_cast<const float4 *>(rowsum + r0);
          const float f = -Epi<BPW>::bias;
          cz[0] = f * rs.x; cz[1] = f * rs.y; cz[2] = f * rs.z; cz[3] = f * rs.w;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t base = wbase + (32 * (a - a0) + 8 * q + 4 * p) * SB + (32 * t + c) * ES;
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = fmaf(acc[a][t][4 * q + j], pt[t], pt[t] * cz[j]);
          if constexpr (OUT_BF16) {
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
              const f32x2_t f2 = {v[j], v[j + 1]};
              const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2, bf16x2_t));
              lds_st16(base + j * SB, h);
              lds_st16(base + (j + 1) * SB, h >> 16);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) lds_stf(base + j * SB, v[j]);
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 32 * CH / RPI; ++it) {
      const int rl = it * RPI + lane / CPR, pc = lane % CPR;
      const uint4 v = lds128(wbase + rl * SB + pc * 16);
      const int64_t r = m0 + 32 * a0 + rl;
      const int64_t col = n0 + pc * EPP;
      if (r < m) {
        uint8_t *dst = reinterpret_cast<uint8_t *>(out) + ((size_t)r * n + col) * ES;
        if (vec && col + EPP <= n) {
          *reinterpret_cast<uint4 *>(dst) = v;
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < EPP; ++e) {
            if (col + e < n) {
              if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(dst)[e] = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
              else reinterpret_cast<uint32_t *>(dst)[e] = w[e];
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// Issue pattern of one MFMA block of the decode-GEMM: 16 rounds of one MFMA
// followed by up to D LDS reads, V VALU operations, W LDS writes and M
// global loads. A wave issues in order and each MFMA 32x32x16 keeps the
// matrix core busy for 32 cycles, so the decode work placed between two
// MFMAs runs in their shadow instead of after a run of back-to-back MFMAs.
template <int V, int D, int W = 0, int M = 0>
__device__ __forceinline__ void gm_interleave16() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if constexpr (W > 0) __builtin_amdgcn_sched_group_barrier(0x200, W, 0);
    if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(0x020, M, 0);
  }
}

template <int BPW, bool G4, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1)
gemm_bf16(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const uint16_t *xt,
          const float *rowsum, int64_t m, int64_t n, int64_t k, float post, const float *row_scale,
          void *out, int vec, int64_t mblocks, int64_t tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t *As0 = reinterpret_cast<uint16_t *>(lds + lds_table_bytes<BPW>());
  uint16_t *As1 = As0 + GM_BM * GM_LDA;
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous range of tiles (m-block fastest) so the workgroups that
  // share an L2 share weight rows and walk the same x~ k-window together.
  int64_t tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int64_t m0 = (tile % mblocks) * GM_BM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, p = lane >> 5;
  const int64_t n0 = (tile / mblocks) * GM_BN + 64 * wave;
  const int64_t G = k / 8;
  const int64_t S = (k + GM_BK - 1) / GM_BK;

  auto load_a = [&](int64_t s, uint4 (&ra)[8]) { gm_load_a(xt, m, k, m0, s, ra); };
  auto load_idx = [&](int64_t s, uint2 (&a)[2], uint2 (&b)[2]) {
    gm_load_idx<BPW, G4>(idx1, idx2, n, G, n0, c, p, s, a, b);
  };

  load_tables<BPW>(lds, blob);
  uint4 ra[8];
  load_a(0, ra);
  uint2 i1[2], i2[2], j1[2], j2[2];
  load_idx(0, i1, i2);
  tables_landed();                                   // tables, x~ tile 0, step-0 indices
  gm_store_a(As0, ra, k);
  // indices of step 1, then x~ tile 1: the same issue order as in the loop,
  // so that the loop-entry wait for the indices does not cover the tile
  load_idx(min((int64_t)1, S - 1), j1, j2);
  load_a(min((int64_t)1, S - 1), ra);
  __syncthreads();                                   // tables and x~ tile 0 in LDS

  f32x16 acc[8][2];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][t][e] = 0.f;

  // Software pipeline: the weights of step s + 1 are decoded while the MFMAs
  // of step s run. A wave issues in order and each SIMD holds one wave, so the
  // decode of the 8 groups is split into phases spread over the four MFMA
  // blocks (records, half-vector offsets and reads, combine), and each
  // phase's LDS reads have MFMAs to hide behind instead of stalling the wave.
  // B operands of a step: group g = 4 t + u in register set [g]; two sets,
  // the step's own and the next step's (decoded while this one runs), which
  // trade places from one step to the next (the loop is unrolled by two).
  uint4 B0[8], B1[8];
  gm_dec_idx<BPW>(i1, i2);
#pragma unroll
  for (int g = 0; g < 8; ++g) B0[g] = gm_decode_one<BPW>(i1, i2, g >> 2, g & 3, lds);
#pragma unroll
  for (int t = 0; t < 2; ++t) { i1[t] = j1[t]; i2[t] = j2[t]; }

  // A operands of MFMA block u sit in set u & 1 and those of block u + 1 are
  // read while block u runs; block 3 reads block 0 of the next tile, so the
  // step's barrier sits between blocks 2 and 3: by then every wave has read
  // its last operands of tile s and written tile s + 1 (into the buffer tile
  // s - 1 used), and after it block 3's MFMAs cover the first reads of tile
  // s + 1. Nothing waits for an operand read at the start of a step.
  uint4 A0[8], A1[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) A0[a] = *reinterpret_cast<const uint4 *>(As0 + (32 * a + c) * GM_LDA + 32 * p);

  auto kstep = [&](int64_t s, const uint4 (&bc)[8], uint4 (&bn)[8]) {
    const uint16_t *Acur = (s & 1) ? As1 : As0;
    uint16_t *Anext = (s & 1) ? As0 : As1;
    // indices of step s + 1 (group g = 4 t + u), as i' = i - 1 mod 2^16
    uint32_t q1[8], q2[8];
    {
      uint2 d1[2] = {i1[0], i1[1]}, d2[2] = {i2[0], i2[1]};
      gm_dec_idx<BPW>(d1, d2);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int t = g >> 2, u = g & 3;
        q1[g] = ((u < 2 ? d1[t].x : d1[t].y) >> (16 * (u & 1))) & 0xFFFFu;
        if constexpr (BPW == 3) q2[g] = (d2[t].x >> (8 * u)) & 0xFFu;
        else if constexpr (BPW == 4) q2[g] = ((u < 2 ? d2[t].x : d2[t].y) >> (16 * (u & 1))) & 0xFFFFu;
        else q2[g] = 0u;
      }
    }
    load_idx(min(s + 2, S - 1), i1, i2);

    auto mfma_block = [&](int u, const uint4 (&av)[8], uint4 (&an)[8]) {
#pragma unroll
      for (int a = 0; a < 8; ++a)
        an[a] = u < 3 ? *reinterpret_cast<const uint4 *>(Acur + (32 * a + c) * GM_LDA + 32 * p + 8 * (u + 1))
                      : *reinterpret_cast<const uint4 *>(Anext + (32 * a + c) * GM_LDA + 32 * p);
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        acc[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                            __builtin_bit_cast(bf16x8, bc[u]), acc[a][0], 0, 0, 0);
        acc[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                            __builtin_bit_cast(bf16x8, bc[4 + u]), acc[a][1], 0, 0, 0);
      }
    };

    // The decode of step s + 1, staggered over the four MFMA blocks: the
    // records of all 8 groups in block 0; the half-vector offsets (about
    // seven VALU operations per table walk) and reads of groups 0-3 in block
    // 1 and of groups 4-7 in block 2; the combine of groups 0-3 in block 2
    // and of groups 4-7 in block 3. x~ tile s + 1 goes to LDS and tile s + 2
    // is requested during block 2.
    constexpr int NW = BPW == 4 ? 2 : 1;            // table walks per group
    constexpr int LA = 1;                           // address arithmetic of a pointer-based load
    Dec8<BPW, false> D;
    D.p1(q1, q2);
    mfma_block(0, A0, A1);
    gm_interleave16<2 + LA, (8 * NW + (BPW == 3 ? 8 : 0) + 8 + 15) / 16>();
    __builtin_amdgcn_sched_barrier(0);
    D.template p2<0, 4>(q1, q2);
    mfma_block(1, A1, A0);
    gm_interleave16<(28 * NW + 15) / 16, (8 * NW + 8 + 15) / 16>();
    __builtin_amdgcn_sched_barrier(0);
    D.template p2<4, 8>(q1, q2);
    D.template p3<0, 4>(bn);
    gm_store_a(Anext, ra, k - GM_BK * (s + 1));     // tile s + 1 (unused past the end)
    load_a(min(s + 2, S - 1), ra);
    mfma_block(2, A0, A1);
    gm_interleave16<(28 * NW + (BPW == 2 ? 0 : 16) + 15) / 16 + LA, (8 * NW + 8 + 15) / 16, 1, 1>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    D.template p3<4, 8>(bn);
    mfma_block(3, A1, A0);
    gm_interleave16<1, 1>();
    __builtin_amdgcn_sched_barrier(0);
  };
  int64_t s = 0;
  for (; s + 1 < S; s += 2) {
    kstep(s, B0, B1);
    kstep(s + 1, B1, B0);
  }
  if (s < S) kstep(s, B0, B1);
  __syncthreads();                                   // the epilogue reuses the x~ buffers
  gm_epilogue<BPW, OUT_BF16>(acc, rowsum, post, row_scale, out, m, n, m0, n0, lane, wave, vec != 0);
}

// Issue pattern of N MFMAs with up to V VALU, D LDS-read, W LDS-write and M
// global-load instructions placed after each (gm_interleave16 for any N).
template <int N, int V, int D, int W = 0, int M = 0>
__device__ __forceinline__ void gm_interleave() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if constexpr (W > 0) __builtin_amdgcn_sched_group_barrier(0x200, W, 0);
    if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(0x020, M, 0);
  }
}

// ---------------------------------------------------------------- 8-wave decode-GEMM
// gemm8_bf16 (m > 16, k a multiple of 64): the tile, the x~ staging and the
// epilogue of gemm_bf16 with 8 waves, two per SIMD. Wave w owns weight rows
// n0 + 32 w .. + 31 for all 256 activation rows (8 MFMA 32x32x16 tiles, 128
// accumulators), so every weight is still decoded once per workgroup, while
// each SIMD now interleaves two instruction streams: one wave's decode
// (VALU and table reads) and operand reads issue while the other wave's
// MFMAs run. Lane (c, p) of a wave decodes groups 8 s + 4 p + u (u = 0..3)
// of weight row n0 + 32 w + c: the B operand of MFMA k-step u, and the x~
// columns the A operands read for that step. A k-step is eight half-blocks
// of four MFMAs (k-step u = h >> 1, activation tiles 4 (h & 1) .. + 3); the
// operands of half-block h + 1 are read during h, and the last half-block
// reads the first of the next x~ tile, after the step's barrier.
constexpr int G8_THREADS = 512;
// LDS the 8-wave epilogue stages through: per wave 4 blocks of 32 rows of 32
// bf16 values padded to 80 bytes (the float32 form, 2 blocks of 144-byte
// rows, is smaller)
constexpr size_t G8_EPI_BYTES = (size_t)(G8_THREADS / 64) * 4 * 32 * (32 * 2 + 16);
static_assert(lds_table_bytes<2>() + 2 * GM_A_BYTES >= G8_EPI_BYTES, "decode-GEMM LDS holds the epilogue");

struct G8Buf {
  __amdgpu_buffer_rsrc_t xa, i1, i2;
  uint32_t va;           // x~ piece 0 of this thread; piece u is 64 u rows further
  uint32_t vi, vi8;      // this lane's index row (2-byte, 1-byte planes)
  int sa;                // bytes of 64 x~ rows
};

template <int BPW>
__device__ __forceinline__ void g8_buf_init(G8Buf &b, const uint16_t *idx1, const void *idx2, const uint16_t *xt,
                                            int64_t m, int64_t n, int64_t k, int64_t m0, int64_t nrow0, int c,
                                            int p) {
  const int64_t G = k / 8;
  const int64_t rows_a = min(m - m0, (int64_t)GM_BM);
  b.xa = __builtin_amdgcn_make_buffer_rsrc((void *)(xt + m0 * k), 0, (int)(rows_a * k * 2), 0x00020000);
  const int64_t rows_w = max(min(n - nrow0, (int64_t)32), (int64_t)0);
  b.i1 = __builtin_amdgcn_make_buffer_rsrc((void *)(idx1 + nrow0 * G), 0, (int)(rows_w * G * 2), 0x00020000);
  if constexpr (BPW == 3)
    b.i2 = __builtin_amdgcn_make_buffer_rsrc((void *)(reinterpret_cast<const uint8_t *>(idx2) + nrow0 * G), 0,
                                             (int)(rows_w * G), 0x00020000);
  else if constexpr (BPW == 4)
    b.i2 = __builtin_amdgcn_make_buffer_rsrc((void *)(reinterpret_cast<const uint16_t *>(idx2) + nrow0 * G), 0,
                                             (int)(rows_w * G * 2), 0x00020000);
  else
    b.i2 = b.i1;
  b.va = (uint32_t)((threadIdx.x >> 3) * k * 2 + 16 * (threadIdx.x & 7));
  b.vi = (uint32_t)(c * G * 2 + 8 * p);
  b.vi8 = (uint32_t)(c * G + 4 * p);
  b.sa = (int)(64 * k * 2);
}

__device__ __forceinline__ void g8_load_a(const G8Buf &b, int64_t s, uint4 (&ra)[4]) {
  const int so = (int)(2 * GM_BK * s);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    ra[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b.xa, b.va, so + u * b.sa, 0));
}

// indices of k-step s as stored (i1: 4 stage-1 indices; i2: stage 2)
template <int BPW>
__device__ __forceinline__ void g8_load_idx(const G8Buf &b, int64_t s, uint2 &i1, uint2 &i2) {
  i1 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(b.i1, b.vi, (int)(16 * s), 0));
  if constexpr (BPW == 3) i2 = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(b.i2, b.vi8, (int)(8 * s), 0), 0u);
  else if constexpr (BPW == 4) i2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(b.i2, b.vi, (int)(16 * s), 0));
  else i2 = make_uint2(0u, 0u);
}

// stored indices -> decode inputs of groups u = 0..3 (as decode_ip takes them)
template <int BPW>
__device__ __forceinline__ void g8_split(uint2 i1, uint2 i2, uint32_t (&q1)[8], uint32_t (&q2)[8]) {
  const uint2 d1 = make_uint2(pk_dec16(i1.x), pk_dec16(i1.y));
  const uint2 d2 = BPW == 4 ? make_uint2(pk_dec16(i2.x), pk_dec16(i2.y)) : i2;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    q1[u] = ((u < 2 ? d1.x : d1.y) >> (16 * (u & 1))) & 0xFFFFu;
    if constexpr (BPW == 3) q2[u] = (d2.x >> (8 * u)) & 0xFFu;
    else if constexpr (BPW == 4) q2[u] = ((u < 2 ? d2.x : d2.y) >> (16 * (u & 1))) & 0xFFFFu;
    else q2[u] = 0u;
  }
}

// k split of the decode-GEMM for layers with fewer 256 x 256 tiles than CUs
// and long rows (the 3072 x 12288 down projection at 4,096 tokens: 192 tiles
// on 256 CUs, 192 k-steps). Tile t's k-steps 0 .. s_main - 1 run on
// workgroup t (its main part), the remaining ones (its remainder) on
// workgroup tiles + t; the remainders start on the CUs the main parts leave
// free and follow one another there (3 on each at 192 tiles: the main parts
// run 146 of 192 steps, the remainders 46). The two parts of a tile meet through float32
// partial sums in the workspace and a counter in the control words; neither
// part ever waits for the other: a part that finds the other's partial
// complete adds it and runs the epilogue, otherwise it publishes its own
// partial (write-through stores, completed before the counter is taken) and
// the other part, arriving second, finishes the tile and clears the counter.
// The main part checks the counter before publishing, so a remainder that
// finished earlier costs it no partial of its own.
struct G8Split {
  float *part;            // [tiles][2][512 threads x 128 accumulators] (main part, remainder)
  unsigned int *ctrl;     // control words: tile t's counter in a dword the single-launch layer leaves unused
  int64_t s_main;         // k-steps of a main part (even)
};

// counter of tile t: dwords 1 .. 63 of the sixteen 256-byte control lines
// (dword 0 of each is a group counter of the single-launch layer), t < 1008
__device__ __forceinline__ unsigned int *g8_tile_counter(unsigned int *ctrl, int64_t t) {
  return ctrl + 64 * (t % 16) + 1 + t / 16;
}

// Join the two parts of tile t (every thread of the workgroup calls it):
// returns true when acc now holds the tile's whole sum (this part finishes
// the tile), false when this part has published its partial for the other.
__device__ __forceinline__ bool g8_split_join(f32x16 (&acc)[8][1], const G8Split &sp, int64_t t, bool main_part,
                                              int *flag) {
  unsigned int *cnt = g8_tile_counter(sp.ctrl, t);
  const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(sp.part + ((size_t)t * 2 + (main_part ? 0 : 1)) * 65536), 0, 65536 * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t other = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(sp.part + ((size_t)t * 2 + (main_part ? 1 : 0)) * 65536), 0, 65536 * 4, 0x00020000);
  // accumulator block (a, e) of thread tid at floats 4 ((4 a + e) 512 + tid): 16 bytes a thread, whole
  // 2 KiB runs a wave
  int done = 0;
  if (main_part) {
    if (threadIdx.x == 0) *flag = (int)__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    done = *flag;
    __syncthreads();
  }
  if (!done) {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4 v = {acc[a][0][4 * e], acc[a][0][4 * e + 1], acc[a][0][4 * e + 2], acc[a][0][4 * e + 3]};
        // sc1: written through to the memory side, where the other part reads it
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), mine,
                                               16 * ((4 * a + e) * G8_THREADS + (int)threadIdx.x), 0, 16);
      }
    __builtin_amdgcn_s_waitcnt(0);                   // the partial is at the memory side
    __syncthreads();
    if (threadIdx.x == 0) *flag = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    done = *flag;
    __syncthreads();
    if (!done) return false;                         // first: the other part finishes the tile
  }
  // one accumulator tile (16 floats) in flight at a time: the k-loop's
  // registers are free here, but all 128 loads at once would not fit
#pragma unroll
  for (int a = 0; a < 8; ++a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    other, 16 * ((4 * a + e) * G8_THREADS + (int)threadIdx.x), 0, 16));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[a][0][4 * e + j] += v[j];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <int BPW, bool OUT_BF16, bool SPLIT = false>
__global__ void __launch_bounds__(G8_THREADS, 1)
gemm8_bf16(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const uint16_t *xt,
           const float *rowsum, int64_t m, int64_t n, int64_t k, float post, const float *row_scale,
           void *out, int vec, int64_t mblocks, int64_t tiles, G8Split sp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t *As0 = reinterpret_cast<uint16_t *>(lds + lds_table_bytes<BPW>());
  uint16_t *As1 = As0 + GM_BM * GM_LDA;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, p = lane >> 5;
  const int64_t S = k / GM_BK;
  // work: workgroup b < tiles runs a main part (unsplit: the whole tile),
  // workgroup tiles + t the remainder of tile t
  const bool main_part = !SPLIT || (int64_t)blockIdx.x < tiles;
  const int64_t s0 = SPLIT && !main_part ? sp.s_main : 0, s1 = SPLIT && main_part ? sp.s_main : S;
  // XCD-aware tile order, as in gemm_bf16
  int64_t tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  if (SPLIT && !main_part) tile = (int64_t)blockIdx.x - tiles;
  const int64_t m0 = (tile % mblocks) * GM_BM;
  const int64_t n0 = (tile / mblocks) * GM_BN + 32 * wave;

  G8Buf gb;
  g8_buf_init<BPW>(gb, idx1, idx2, xt, m, n, k, m0, n0, c, p);
  // x~ piece u of this thread: row (tid >> 3) + 64 u, 16-byte column tid & 7
  auto store_a = [&](uint16_t *As, const uint4 (&ra)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = threadIdx.x + G8_THREADS * u;
      *reinterpret_cast<uint4 *>(As + (pc >> 3) * GM_LDA + 8 * (pc & 7)) = ra[u];
    }
  };

  load_tables<BPW, G8_THREADS>(lds, blob);
  uint4 ra[4];
  g8_load_a(gb, s0, ra);
  uint2 i1, i2, j1, j2;
  g8_load_idx<BPW>(gb, s0, i1, i2);
  tables_landed();                                   // tables, x~ tile s0, step-s0 indices
  store_a(As0, ra);                                  // (s0 is even)
  g8_load_idx<BPW>(gb, min(s0 + 1, s1 - 1), j1, j2);
  g8_load_a(gb, min(s0 + 1, s1 - 1), ra);
  __syncthreads();                                   // tables and x~ tile s0 in LDS

  f32x16 acc[8][1];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[a][0][e] = 0.f;

  uint4 B0[8], B1[8];                                // groups u = 0..3 used
  {
    uint32_t q1[8], q2[8];
    g8_split<BPW>(i1, i2, q1, q2);
#pragma unroll
    for (int u = 0; u < 4; ++u) B0[u] = decode_ip<BPW>(q1[u], q2[u]);
  }
  i1 = j1;
  i2 = j2;

  uint4 H0[4], H1[4];                                // A operands of even / odd half-blocks
#pragma unroll
  for (int a = 0; a < 4; ++a) H0[a] = *reinterpret_cast<const uint4 *>(As0 + (32 * a + c) * GM_LDA + 32 * p);

  auto kstep = [&](int64_t s, const uint4 (&bc)[8], uint4 (&bn)[8]) {
    const uint16_t *Acur = (s & 1) ? As1 : As0;
    uint16_t *Anext = (s & 1) ? As0 : As1;
    uint32_t q1[8], q2[8];
    g8_split<BPW>(i1, i2, q1, q2);                   // indices of step s + 1
    g8_load_idx<BPW>(gb, min(s + 2, s1 - 1), i1, i2);

    // half-block h: MFMAs of k-step u = h >> 1 on activation tiles 4 (h & 1) + a,
    // reading the operands of half-block h + 1 (of the next tile for h = 7)
    auto half = [&](int h, const uint4 (&av)[4], uint4 (&an)[4]) {
      const int hn = h + 1, un = (hn >> 1) & 3, tn = 4 * (hn & 1);
      const uint16_t *Ab = h < 7 ? Acur : Anext;
#pragma unroll
      for (int a = 0; a < 4; ++a)
        an[a] = *reinterpret_cast<const uint4 *>(Ab + (32 * (tn + a) + c) * GM_LDA + 32 * p + 8 * un);
      const int u = h >> 1, t0 = 4 * (h & 1);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        acc[t0 + a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                                 __builtin_bit_cast(bf16x8, bc[u]), acc[t0 + a][0],
                                                                 0, 0, 0);
    };
    constexpr int NW = BPW == 4 ? 2 : 1;             // table walks per group
    Dec8<BPW, true> D;
    D.template p1<0, 4>(q1, q2);
    half(0, H0, H1);
    gm_interleave<4, 3, (4 * NW + (BPW == 3 ? 4 : 0) + 4 + 3) / 4>();
    __builtin_amdgcn_sched_barrier(0);
    D.template p2<0, 2>(q1, q2);
    half(1, H1, H0);
    gm_interleave<4, (14 * NW + 3) / 4, (4 * NW + 4 + 3) / 4>();
    __builtin_amdgcn_sched_barrier(0);
    D.template p2<2, 4>(q1, q2);
    half(2, H0, H1);
    gm_interleave<4, (14 * NW + 3) / 4, (4 * NW + 4 + 3) / 4>();
    __builtin_amdgcn_sched_barrier(0);
    D.template p3<0, 2>(bn);
    half(3, H1, H0);
    gm_interleave<4, 2, 1>();
    __builtin_amdgcn_sched_barrier(0);
    D.template p3<2, 4>(bn);
    store_a(Anext, ra);                              // tile s + 1 (unused past the end)
    half(4, H0, H1);
    gm_interleave<4, 2, 1, 1>();
    __builtin_amdgcn_sched_barrier(0);
    g8_load_a(gb, min(s + 2, s1 - 1), ra);
    half(5, H1, H0);
    gm_interleave<4, 0, 1, 0, 1>();
    __builtin_amdgcn_sched_barrier(0);
    half(6, H0, H1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    half(7, H1, H0);
    __builtin_amdgcn_sched_barrier(0);
  };
  int64_t s = s0;
  for (; s + 1 < s1; s += 2) {
    kstep(s, B0, B1);
    kstep(s + 1, B1, B0);
  }
  if (s < s1) kstep(s, B0, B1);
  __syncthreads();                                   // the epilogue reuses the x~ buffers
  if constexpr (SPLIT) {
    // the join's flag word lives in the x~ buffer, free after the k-loop
    if (!g8_split_join(acc, sp, tile, main_part, reinterpret_cast<int *>(As0))) return;
  }
  gm_epilogue<BPW, OUT_BF16, 1>(acc, rowsum, post, row_scale, out, m, n, m0, n0, lane, wave, vec != 0);
}

// Dense GEMM z = post * x~ W^T on bf16 weights in memory [n][k] (the
// entropy-coded layers' decoded weights), k a multiple of 64: 256 x 256
// tiles with both operand tiles double-buffered in LDS ([256][64 + 8] each)
// and 4 waves in a 2 x 2 grid of 128 x 128 wave tiles (4 x 4 MFMA 32x32x16
// tiles, 256 accumulators), so every operand read from LDS feeds four MFMAs.
// Tiles are fetched with buffer loads at fixed per-thread offsets (the step is
// the scalar offset; rows past m or n read as zeros) one step ahead into
// registers and written to LDS during the step before their use; the step's
// barrier sits before the last MFMA block, whose MFMAs cover the first
// operand reads of the next tile (as in gemm_bf16).
template <bool OUT_BF16>
__global__ void __launch_bounds__(256, 1)
gemm_w2_bf16(const uint16_t *w, const uint16_t *xt, int64_t m, int64_t n, int64_t k, float post, void *out,
             int vec, int64_t mblocks, int64_t tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t *As0 = reinterpret_cast<uint16_t *>(lds);
  uint16_t *As1 = As0 + GM_BM * GM_LDA;
  uint16_t *Bs0 = As1 + GM_BM * GM_LDA;
  uint16_t *Bs1 = Bs0 + GM_BN * GM_LDA;
  int64_t tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int64_t m0 = (tile % mblocks) * GM_BM;
  const int64_t nb0 = (tile / mblocks) * GM_BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, p = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;            // wave tile: rows 128 wm, columns 128 wn
  const int64_t S = k / GM_BK;

  const int64_t rows_a = min(m - m0, (int64_t)GM_BM), rows_w = min(n - nb0, (int64_t)GM_BN);
  const __amdgpu_buffer_rsrc_t ra_rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(xt + m0 * k), 0, (int)(rows_a * k * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb_rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(w + nb0 * k), 0, (int)(rows_w * k * 2), 0x00020000);
  // piece u of this thread: tile row (tid >> 3) + 32 u, 16-byte column tid & 7
  const uint32_t voff = (uint32_t)((threadIdx.x >> 3) * k * 2 + 16 * (threadIdx.x & 7));
  const int s32 = (int)(32 * k * 2);
  auto load = [&](const __amdgpu_buffer_rsrc_t &rs, int64_t st, uint4 (&r)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      r[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (int)(2 * GM_BK * st) + u * s32, 0));
  };
  auto store = [&](uint16_t *T, const uint4 (&r)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pc = threadIdx.x + 256 * u;
      *reinterpret_cast<uint4 *>(T + (pc >> 3) * GM_LDA + 8 * (pc & 7)) = r[u];
    }
  };

  uint4 ra[8], rb[8];
  load(ra_rs, 0, ra);
  load(rb_rs, 0, rb);
  store(As0, ra);
  store(Bs0, rb);
  load(ra_rs, min((int64_t)1, S - 1), ra);
  load(rb_rs, min((int64_t)1, S - 1), rb);
  __syncthreads();

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][t][e] = 0.f;

  // operands of MFMA block u (k-step sub-step u): A rows 128 wm + 32 a + c,
  // B rows 128 wn + 32 t + c, inputs 32 p + 8 u .. + 7 (the k order inside a
  // step is a permutation shared by A and B)
  auto rd = [&](const uint16_t *T, int base, int u, uint4 (&v)[4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) v[a] = *reinterpret_cast<const uint4 *>(T + (base + 32 * a + c) * GM_LDA + 32 * p + 8 * u);
  };
  uint4 A0[4], A1[4], B0[4], B1[4];
  rd(As0, 128 * wm, 0, A0);
  rd(Bs0, 128 * wn, 0, B0);

  auto kstep = [&](int64_t st) {
    const uint16_t *Acur = (st & 1) ? As1 : As0, *Bcur = (st & 1) ? Bs1 : Bs0;
    uint16_t *Anext = (st & 1) ? As0 : As1, *Bnext = (st & 1) ? Bs0 : Bs1;
    auto block = [&](int u, const uint4 (&av)[4], const uint4 (&bv)[4], uint4 (&an)[4], uint4 (&bn)[4]) {
      if (u < 3) {
        rd(Acur, 128 * wm, u + 1, an);
        rd(Bcur, 128 * wn, u + 1, bn);
      } else {
        rd(Anext, 128 * wm, 0, an);
        rd(Bnext, 128 * wn, 0, bn);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                              __builtin_bit_cast(bf16x8, bv[t]), acc[a][t], 0, 0, 0);
    };
    block(0, A0, B0, A1, B1);
    gm_interleave16<0, 1>();
    __builtin_amdgcn_sched_barrier(0);
    store(Anext, ra);                                // tiles st + 1 (unused past the end)
    load(ra_rs, min(st + 2, S - 1), ra);
    block(1, A1, B1, A0, B0);
    gm_interleave16<0, 1, 1, 1>();
    __builtin_amdgcn_sched_barrier(0);
    store(Bnext, rb);
    load(rb_rs, min(st + 2, S - 1), rb);
    block(2, A0, B0, A1, B1);
    gm_interleave16<0, 1, 1, 1>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    block(3, A1, B1, A0, B0);
    gm_interleave16<0, 1>();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int64_t st = 0; st < S; ++st) kstep(st);
  __syncthreads();                                   // the epilogue reuses the operand buffers
  gm_epilogue<2, OUT_BF16, 4, 4>(acc, nullptr, post, nullptr, out, m, n, m0 + 128 * wm, nb0 + 128 * wn, lane, wave,
                                 vec != 0);
}

// Dense GEMM z = post * x~ W^T with the weights already in memory as bf16
// [n][k] row-major (the entropy-coded layers' decoded weights): the tiling,
// x~ staging and epilogue of gemm_bf16. The 256 x 64 weight tile of a step
// has the shape of the x~ tile, so it is staged the same way (loaded into
// registers one step ahead, stored to a second double-buffered LDS tile);
// in MFMA block u, lane (c, p) reads inputs 32 p + 8 u .. + 7 of its weight
// row, the order in which it reads its A operands (the k order inside a step
// is a permutation shared by A and B). Past k both tiles are zero.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256, 1)
gemm_w_bf16_lds(const uint16_t *w, const uint16_t *xt, int64_t m, int64_t n, int64_t k, float post, void *out,
            int vec, int64_t mblocks, int64_t tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t *As0 = reinterpret_cast<uint16_t *>(lds);
  uint16_t *As1 = As0 + GM_BM * GM_LDA;
  uint16_t *Bs0 = As1 + GM_BM * GM_LDA;
  uint16_t *Bs1 = Bs0 + GM_BN * GM_LDA;
  int64_t tile = blockIdx.x;
  if (tiles % 8 == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int64_t m0 = (tile % mblocks) * GM_BM;
  const int64_t nb0 = (tile / mblocks) * GM_BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, p = lane >> 5;
  const int64_t n0 = nb0 + 64 * wave;
  const int64_t S = (k + GM_BK - 1) / GM_BK;

  uint4 ra[8], rb[8];
  gm_load_a(xt, m, k, m0, 0, ra);
  gm_load_a(w, n, k, nb0, 0, rb);
  gm_store_a(As0, ra, k);
  gm_store_a(Bs0, rb, k);
  gm_load_a(xt, m, k, m0, min((int64_t)1, S - 1), ra);
  gm_load_a(w, n, k, nb0, min((int64_t)1, S - 1), rb);
  __syncthreads();

  f32x16 acc[8][2];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][t][e] = 0.f;

  // One k-step: four MFMA blocks (sub-steps u of 16 inputs); the A and B
  // operands of block u + 1 are read from LDS while block u runs, into the
  // other of two register sets (no copies), and the reads are spread between
  // the MFMAs; the next tiles go to LDS and the ones after them are loaded
  // during the last block.
  for (int64_t st = 0; st < S; ++st) {
    const uint16_t *Acur = (st & 1) ? As1 : As0;
    const uint16_t *Bcur = ((st & 1) ? Bs1 : Bs0) + (64 * wave) * GM_LDA;
    uint4 A0[8], A1[8], B0[2], B1[2];
#pragma unroll
    for (int a = 0; a < 8; ++a) A0[a] = *reinterpret_cast<const uint4 *>(Acur + (32 * a + c) * GM_LDA + 32 * p);
#pragma unroll
    for (int t = 0; t < 2; ++t) B0[t] = *reinterpret_cast<const uint4 *>(Bcur + (32 * t + c) * GM_LDA + 32 * p);
    auto block = [&](int u, const uint4 (&av)[8], const uint4 (&bv)[2], uint4 (&an)[8], uint4 (&bn)[2]) {
      if (u < 3) {
#pragma unroll
        for (int a = 0; a < 8; ++a)
          an[a] = *reinterpret_cast<const uint4 *>(Acur + (32 * a + c) * GM_LDA + 32 * p + 8 * (u + 1));
#pragma unroll
        for (int t = 0; t < 2; ++t)
          bn[t] = *reinterpret_cast<const uint4 *>(Bcur + (32 * t + c) * GM_LDA + 32 * p + 8 * (u + 1));
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        acc[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                            __builtin_bit_cast(bf16x8, bv[0]), acc[a][0], 0, 0, 0);
        acc[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                            __builtin_bit_cast(bf16x8, bv[1]), acc[a][1], 0, 0, 0);
      }
    };
    block(0, A0, B0, A1, B1);
    gm_interleave16<0, 1>();
    __builtin_amdgcn_sched_barrier(0);
    block(1, A1, B1, A0, B0);
    gm_interleave16<0, 1>();
    __builtin_amdgcn_sched_barrier(0);
    block(2, A0, B0, A1, B1);
    gm_interleave16<0, 1>();
    __builtin_amdgcn_sched_barrier(0);
    block(3, A1, B1, A0, B0);
    const int64_t kv = k - GM_BK * (st + 1);
    gm_store_a((st & 1) ? As0 : As1, ra, kv);          // tiles st + 1 (unused past the end)
    gm_store_a((st & 1) ? Bs0 : Bs1, rb, kv);
    gm_load_a(xt, m, k, m0, min(st + 2, S - 1), ra);
    gm_load_a(w, n, k, nb0, min(st + 2, S - 1), rb);
    gm_interleave16<1, 0, 1, 1>();
    __syncthreads();
  }
  gm_epilogue<2, OUT_BF16>(acc, nullptr, post, nullptr, out, m, n, m0, n0, lane, wave, vec != 0);
}

// Dense GEMV for m <= 16 on weights in memory (bf16 [n][k]): one 16-row
// weight tile per workgroup of 16 waves; the k axis is cut in chunks of 32
// inputs and wave w takes chunks w, w + 16, ... Lane l (row j = l & 15,
// slot q = l >> 4) loads inputs 8 q .. 8 q + 7 of the chunk from x~ row j
// (clamped to m - 1: rows past m feed only outputs that are not stored) and
// from weight row n0 + j, and one MFMA 16x16x32 contracts the chunk (A = x~
// rows, B = weight rows). Four chunks' loads are issued before their MFMAs;
// a partial last chunk (k % 32 != 0) is taken apart, with its weights past k
// zeroed. Partial sums of the 16 waves meet in LDS.
constexpr int GW_WAVES = 16;

__global__ void __launch_bounds__(64 * GW_WAVES)
gemv_w_bf16(const uint16_t *w, const uint16_t *xt, int64_t m, int64_t n, int64_t k, float post, void *out,
            glq_dtype out_dt) {
  __shared__ float red[GW_WAVES * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const uint16_t *xr = xt + (size_t)min((int64_t)j, m - 1) * k + 8 * q;
  const uint16_t *wr = w + (size_t)min(n0 + j, n - 1) * k + 8 * q;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t full = k / 32;
  int64_t c = wave;
  for (; c + 3 * GW_WAVES < full; c += 4 * GW_WAVES) {
    uint4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = *reinterpret_cast<const uint4 *>(xr + 32 * (c + u * GW_WAVES));
      b[u] = *reinterpret_cast<const uint4 *>(wr + 32 * (c + u * GW_WAVES));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, b[u]),
                                                    acc, 0, 0, 0);
  }
  for (; c < full; c += GW_WAVES) {
    const uint4 a = *reinterpret_cast<const uint4 *>(xr + 32 * c);
    const uint4 b = *reinterpret_cast<const uint4 *>(wr + 32 * c);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                  0, 0, 0);
  }
  if ((k & 31) && wave == (int)(full % GW_WAVES)) {       // the partial last chunk
    const int64_t kk = 32 * full + 8 * q;
    const int64_t kc = min(kk, k - 8) - 8 * q;          // clamped, in-bounds load position
    const uint4 a = *reinterpret_cast<const uint4 *>(xr + kc);
    uint4 b = *reinterpret_cast<const uint4 *>(wr + kc);
    if (kk >= k) b = make_uint4(0u, 0u, 0u, 0u);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                  0, 0, 0);
  }
  // D[r][col]: lane holds rows 4 q + t (activation row), column j (weight row)
#pragma unroll
  for (int t = 0; t < 4; ++t) red[(wave * 16 + 4 * q + t) * 16 + j] = acc[t];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int r = threadIdx.x >> 4, col = threadIdx.x & 15;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < GW_WAVES; ++ww) v += red[(ww * 16 + r) * 16 + col];
    if (r < m && n0 + col < n) store_out(out, out_dt, (size_t)r * n + n0 + col, post * v);
  }
}

// ---------------------------------------------------------------- float32 path
// One wave per weight row (grid-stride); lanes split the groups of the row;
// up to 4 activation rows per pass (the host loops over passes).
template <int BPW>
__global__ void __launch_bounds__(256)
gemv_f32(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const float *xt,
         int64_t m0, int64_t mc, int64_t n, int64_t k, float scale, const float *row_scale, void *out,
         glq_dtype out_dt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  load_tables<BPW>(lds, blob);
  tables_landed();
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t G = k / 8;
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); row < n; row += waves) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t g = lane; g < G; g += 64) {
      const uint32_t i1 = idx1[row * G + g];
      const uint32_t i2 = BPW == 2 ? 0u : load_idx2(idx2, row * G + g, BPW);
      const uint4 h = decode_group<BPW>(i1, i2, lds);
      const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = operand_value<BPW>((hw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < mc) {
          const float *xr = xt + (size_t)(m0 + r) * k + 8 * g;
          float sacc = acc[r];
#pragma unroll
          for (int t = 0; t < 8; ++t) sacc = fmaf(v[t], xr[t], sacc);
          acc[r] = sacc;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = acc[r];
      for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
      if (lane == 0 && r < mc)
        store_out(out, out_dt, (size_t)(m0 + r) * n + row, (row_scale ? scale * row_scale[row] : scale) * t);
    }
  }
}

// ------------------------------------------------ entropy-coded lattice layers
// Fused symbol decode and weight reconstruction of the entropy-coded E8
// format ("Transformers Proposes EntroPack Integration ...", first two
// paragraphs; the format is this library's reading, defined in glq.h).
// One wave per coded block: lane l holds the rANS state of the block's lane
// l and all 64 step through their groups' 8 symbols in lockstep. The words a
// step needs are taken from the block's stream in lane order (ballot, then a
// prefix count with mbcnt) out of a per-wave ring of 2048 words in LDS. The
// ring is filled on a fixed schedule: the prologue publishes the first 1024
// words (from the 8-aligned start) and loads 512 more; every round (8 steps)
// ends by publishing the loaded 512 and loading the next 512 (16 bytes per
// lane), so each load has a round to land. The fill position advances by 512
// per round but stays within 1024 words of the (8-aligned) read position:
// then the ring holds a round's words (at most 512) before the round starts
// and never overwrites a word not yet read. Next round's row scale is loaded
// just before the words, so waiting for it leaves the word load in flight.
// The five
// decode tables (slot -> symbol | frequency << 8 | (slot - cumulative) << 20,
// 2048 slots each) are copied to LDS once per
// workgroup with global-to-LDS loads.
constexpr uint32_t kEpLutHdr = 64;                    // vmin[5], padded
constexpr uint32_t kEpLutBytes = 5 * 2048 * 4;        // in LDS at offset 0
constexpr uint32_t kEpRing = 2048;                    // words per wave
constexpr uint32_t ep_lds(uint32_t waves) { return kEpLutBytes + waves * kEpRing * 2; }

typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4_t lds_u128_w;
__device__ __forceinline__ uint32_t lds32(uint32_t addr) {
  return *reinterpret_cast<lds_u32 *>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ void lds_st128(uint32_t addr, uint4 v) {
  u32x4_t t = {v.x, v.y, v.z, v.w};
  *reinterpret_cast<lds_u128_w *>(static_cast<uintptr_t>(addr)) = t;
}

template <bool F32, uint32_t kEpWaves>
__global__ __launch_bounds__(64 * kEpWaves) void ep_decode_k(const uint32_t *__restrict__ states,
                                                   const uint32_t *__restrict__ offsets,
                                                   const uint16_t *__restrict__ words, uint32_t nwords,
                                                   const uint8_t *__restrict__ lut,
                                                   const float *__restrict__ row_scale, float step,
                                                   uint32_t total_groups, uint32_t gpr, uint32_t lane_groups,
                                                   uint32_t nblocks, uint32_t k, void *__restrict__ out) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (uint32_t r = wave; r < kEpLutBytes / 1024; r += kEpWaves)
    __builtin_amdgcn_global_load_lds((glb_void_t *)(lut + kEpLutHdr + 1024 * r + 16 * lane),
                                     (lds_void_t *)(uintptr_t)(1024 * r), 16, 0, 0);
  const int32_t *vm = reinterpret_cast<const int32_t *>(lut);
  const int32_t vm0 = vm[0], vm1 = vm[1], vm2 = vm[2], vm3 = vm[3], vm4 = vm[4];
  tables_landed();
  __syncthreads();
  const uint32_t blk = blockIdx.x * kEpWaves + wave;
  if (blk >= nblocks) return;

  const uint32_t ring = kEpLutBytes + wave * kEpRing * 2;   // this wave's ring (bytes)
  const uint32_t bg = 64 * lane_groups;
  const uint32_t g0 = blk * bg;
  const uint32_t ng = min(bg, total_groups - g0);
  uint32_t x = states[(size_t)blk * 64 + lane];
  uint32_t pos = __builtin_amdgcn_readfirstlane(offsets[blk]);   // next word (wave-uniform)
  // 16-byte loads of 8 words at 8-aligned positions, clamped to the last
  // 8-aligned start below nwords (the buffer is padded to a multiple of 8
  // words, at least 8); positions past the stream get stale words, which a
  // valid stream never reads
  const uint32_t lastq = nwords > 0 ? ((nwords - 1) & ~7u) : 0u;
  auto ld8 = [&](uint32_t at) -> uint4 {
    return *reinterpret_cast<const uint4 *>(words + min(at + 8 * lane, lastq));
  };
  // prologue: words [f0, f0 + 1024) published, [f0 + 1024, f0 + 1536) loading
  uint32_t f = pos & ~7u;                             // fill position of pend
  lds_st128(ring + ((f + 8 * lane) & (kEpRing - 1)) * 2, ld8(f));
  lds_st128(ring + ((f + 512 + 8 * lane) & (kEpRing - 1)) * 2, ld8(f + 512));
  // the start state is waited for here: left to the loop, the wait at the
  // loop head would also hold every later round on its last store
  asm volatile("" ::"v"(x));
  f += 1024;
  float rs = row_scale[min(g0 + lane, total_groups - 1) / gpr];   // round 0's row scale
  __builtin_amdgcn_sched_barrier(0);
  uint4 pend = ld8(f);
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t rounds = (ng + 63) / 64;
  for (uint32_t p = 0; p < rounds; ++p) {
    const uint32_t j = p * 64 + lane;
    const bool act = j < ng;
    const uint32_t gi = min(g0 + j, total_groups - 1);
    const uint64_t actm = __builtin_amdgcn_ballot_w64(act);   // lanes with a group this round
    int32_t z[8];
    int32_t b = 0, s7 = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t tb = c == 0 ? 0u : (c < 7 ? 1u + (uint32_t)b : 3u + (uint32_t)b);
      const uint32_t e = lds32(tb * 8192u + (x & 2047u) * 4u);
      // lanes past the block's end decode garbage: they read no words and
      // their values are never stored
      x = ((e >> 8) & 0xFFFu) * (x >> 11) + (e >> 20);
      const int32_t sym = (int32_t)(e & 0xFFu);
      if (c == 0) {
        z[0] = sym + vm0;
        b = z[0] & 1;
        s7 = z[0];
      } else if (c < 7) {
        z[c] = 2 * (sym + (b ? vm2 : vm1)) + b;
        s7 += z[c];
      } else {
        z[7] = 4 * (sym + (b ? vm4 : vm3)) + ((-s7) & 3);
      }
      const bool low = x < 65536u;
      const bool need = act && low;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(low) & actm;
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      const uint32_t wd = lds16(ring + ((pos + below) & (kEpRing - 1)) * 2);
      x = need ? ((x << 16) | wd) : x;
      pos += (uint32_t)__popcll(mask);
    }
    // Stores and the row-scale load are issued by every lane (lanes past the
    // block's end repeat lane 0's store: same bytes, same address), so the
    // count of vector-memory operations per round is fixed and the next
    // round waits for its word load alone, not for this round's stores.
    // Groups are row-major, so group gi's 8 weights start at element 8 gi.
    const float er = __fmul_rn(step, rs);
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = __fmul_rn(er, (float)z[c] * 0.5f);
    // lane 0 is active in every round: its group is g0 + 64 p, and its values
    // are read with readlane(., 0), which (unlike readfirstlane) does not
    // depend on which lanes are enabled where the compiler places it
    const uint32_t gs = act ? gi : g0 + p * 64;
    if constexpr (F32) {
      float u[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[c]), 0));
        u[c] = act ? v[c] : l;
      }
      float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + (size_t)gs * 8);
      dst[0] = make_float4(u[0], u[1], u[2], u[3]);
      dst[1] = make_float4(u[4], u[5], u[6], u[7]);
    } else {
      uint32_t h0 = bf16x2_rne(v[0], v[1]), h1 = bf16x2_rne(v[2], v[3]);
      uint32_t h2 = bf16x2_rne(v[4], v[5]), h3 = bf16x2_rne(v[6], v[7]);
      const uint32_t l0 = __builtin_amdgcn_readlane((int)h0, 0), l1 = __builtin_amdgcn_readlane((int)h1, 0);
      const uint32_t l2 = __builtin_amdgcn_readlane((int)h2, 0), l3 = __builtin_amdgcn_readlane((int)h3, 0);
      h0 = act ? h0 : l0;
      h1 = act ? h1 : l1;
      h2 = act ? h2 : l2;
      h3 = act ? h3 : l3;
      *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + (size_t)gs * 8) = make_uint4(h0, h1, h2, h3);
    }
    // publish the words loaded a round ago; next round's row scale, then
    // the next 512 words (scheduling barriers keep this order: the word load
    // must be the youngest vector-memory operation)
    const uint32_t rsi = min(g0 + j + 64, total_groups - 1) / gpr;
    const uint32_t fn = min(f + 512, (pos & ~7u) + 1024);
    __builtin_amdgcn_sched_barrier(0);
    lds_st128(ring + ((f + 8 * lane) & (kEpRing - 1)) * 2, pend);
    rs = row_scale[rsi];
    __builtin_amdgcn_sched_barrier(0);
    f = fn;
    pend = ld8(f);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The layer product on an entropy-coded weight set at batch 1, fused with
// the decode: the same symbol decode as ep_decode_k (one wave per block, the
// word ring in LDS), but each lane multiplies its group's 8 reconstructed
// weights (float32, exact) with the 8 matching entries of x~ (bf16 [k])
// instead of storing them. A lane keeps the partial sum of its current output
// row in a register; when its next group starts another row (groups run
// row-major) it adds the sum into the wave's row sums in LDS (the rmax rows
// its block touches), and at the end of the block the wave adds those into z
// (float32 [n], zeroed before the launch) with one atomic per row. The
// decoded weights never reach memory. At batch 2 and more the decode-once
// path wins: there every 8 weights would re-read m x 16 bytes of x~ from the
// caches, more than writing W^ as bf16 once and streaming it through the GEMV.
template <uint32_t kEpWaves>
__global__ __launch_bounds__(64 * kEpWaves) void ep_gemv_k(const uint32_t *__restrict__ states,
                                                 const uint32_t *__restrict__ offsets,
                                                 const uint16_t *__restrict__ words, uint32_t nwords,
                                                 const uint8_t *__restrict__ lut,
                                                 const float *__restrict__ row_scale, float step,
                                                 uint32_t total_groups, uint32_t gpr, uint32_t lane_groups,
                                                 uint32_t nblocks, const uint16_t *__restrict__ xt,
                                                 float *__restrict__ z, uint32_t rmax) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (uint32_t r = wave; r < kEpLutBytes / 1024; r += kEpWaves)
    __builtin_amdgcn_global_load_lds((glb_void_t *)(lut + kEpLutHdr + 1024 * r + 16 * lane),
                                     (lds_void_t *)(uintptr_t)(1024 * r), 16, 0, 0);
  const int32_t *vm = reinterpret_cast<const int32_t *>(lut);
  const int32_t vm0 = vm[0], vm1 = vm[1], vm2 = vm[2], vm3 = vm[3], vm4 = vm[4];
  float *racc = reinterpret_cast<float *>(lds + ep_lds(kEpWaves)) + wave * rmax;
  for (uint32_t e = lane; e < rmax; e += 64) racc[e] = 0.0f;
  tables_landed();
  __syncthreads();
  const uint32_t blk = blockIdx.x * kEpWaves + wave;
  if (blk >= nblocks) return;

  const uint32_t ring = kEpLutBytes + wave * kEpRing * 2;   // this wave's ring (bytes)
  const uint32_t bg = 64 * lane_groups;
  const uint32_t g0 = blk * bg;
  const uint32_t ng = min(bg, total_groups - g0);
  const uint32_t rbase = g0 / gpr, rlast = (g0 + ng - 1) / gpr;
  uint32_t x = states[(size_t)blk * 64 + lane];
  uint32_t pos = __builtin_amdgcn_readfirstlane(offsets[blk]);
  const uint32_t lastq = nwords > 0 ? ((nwords - 1) & ~7u) : 0u;
  auto ld8 = [&](uint32_t at) -> uint4 {
    return *reinterpret_cast<const uint4 *>(words + min(at + 8 * lane, lastq));
  };
  uint32_t f = pos & ~7u;
  lds_st128(ring + ((f + 8 * lane) & (kEpRing - 1)) * 2, ld8(f));
  lds_st128(ring + ((f + 512 + 8 * lane) & (kEpRing - 1)) * 2, ld8(f + 512));
  asm volatile("" ::"v"(x));
  f += 1024;
  float rs = row_scale[min(g0 + lane, total_groups - 1) / gpr];
  __builtin_amdgcn_sched_barrier(0);
  uint4 pend = ld8(f);
  __builtin_amdgcn_sched_barrier(0);

  float acc = 0.0f;
  uint32_t cur = 0xFFFFFFFFu;                         // row (relative to rbase) of acc
  const uint32_t rounds = (ng + 63) / 64;
  for (uint32_t p = 0; p < rounds; ++p) {
    const uint32_t j = p * 64 + lane;
    const bool act = j < ng;
    const uint32_t gi = min(g0 + j, total_groups - 1);
    const uint32_t row = gi / gpr, q = gi - row * gpr;
    const uint64_t actm = __builtin_amdgcn_ballot_w64(act);   // lanes with a group this round
    const uint4 xv = *reinterpret_cast<const uint4 *>(xt + 8 * (size_t)q);   // this group's 8 inputs
    int32_t zz[8];
    int32_t b = 0, s7 = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t tb = c == 0 ? 0u : (c < 7 ? 1u + (uint32_t)b : 3u + (uint32_t)b);
      const uint32_t e = lds32(tb * 8192u + (x & 2047u) * 4u);
      x = ((e >> 8) & 0xFFFu) * (x >> 11) + (e >> 20);
      const int32_t sym = (int32_t)(e & 0xFFu);
      if (c == 0) {
        zz[0] = sym + vm0;
        b = zz[0] & 1;
        s7 = zz[0];
      } else if (c < 7) {
        zz[c] = 2 * (sym + (b ? vm2 : vm1)) + b;
        s7 += zz[c];
      } else {
        zz[7] = 4 * (sym + (b ? vm4 : vm3)) + ((-s7) & 3);
      }
      const bool low = x < 65536u;
      const bool need = act && low;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(low) & actm;
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      const uint32_t wd = lds16(ring + ((pos + below) & (kEpRing - 1)) * 2);
      x = need ? ((x << 16) | wd) : x;
      pos += (uint32_t)__popcll(mask);
    }
    const float er = __fmul_rn(step, rs);
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = __fmul_rn(er, (float)zz[c] * 0.5f);
    const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
    float d = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d = fmaf(v[2 * c], __uint_as_float(w4[c] << 16), d);
      d = fmaf(v[2 * c + 1], __uint_as_float(w4[c] & 0xFFFF0000u), d);
    }
    if (act) {
      const uint32_t rr = row - rbase;
      if (rr != cur) {
        if (cur != 0xFFFFFFFFu)
          __hip_atomic_fetch_add(racc + cur, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        acc = 0.0f;
        cur = rr;
      }
      acc += d;
    }
    const uint32_t rsi = min(g0 + j + 64, total_groups - 1) / gpr;
    const uint32_t fn = min(f + 512, (pos & ~7u) + 1024);
    __builtin_amdgcn_sched_barrier(0);
    lds_st128(ring + ((f + 8 * lane) & (kEpRing - 1)) * 2, pend);
    rs = row_scale[rsi];
    __builtin_amdgcn_sched_barrier(0);
    f = fn;
    pend = ld8(f);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (cur != 0xFFFFFFFFu)
    __hip_atomic_fetch_add(racc + cur, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // the wave's LDS atomics are done before its lanes read the sums back
  __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  for (uint32_t rr = lane; rr <= rlast - rbase; rr += 64)
    __hip_atomic_fetch_add(z + rbase + rr, racc[rr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- host helpers
thread_local char g_last_error[256] = "";

int hip_status(hipError_t e, const char *where = "launch") {
  if (e == hipSuccess) return GLQ_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return GLQ_ERR_HIP;
}

// Allow dynamic LDS above the 64 KiB default (gfx950 has 160 KiB per CU).
// The attribute is raised once per kernel (keyed by its address: kernels of
// one signature share a function-pointer type) to the largest size asked.
template <class K>
int allow_lds(K kernel, size_t bytes) {
  if (bytes <= 60 * 1024) return GLQ_OK;
  static std::mutex mu;
  static std::vector<std::pair<const void *, size_t>> granted;
  const void *key = reinterpret_cast<const void *>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (auto &g : granted)
    if (g.first == key) {
      if (g.second >= bytes) return GLQ_OK;
      const int rc = hip_status(hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes),
                                "hipFuncSetAttribute");
      if (rc == GLQ_OK) g.second = bytes;
      return rc;
    }
  const int rc = hip_status(hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes),
                            "hipFuncSetAttribute");
  if (rc == GLQ_OK) granted.emplace_back(key, bytes);
  return rc;
}

constexpr int kMaxLogBlock = 14;   // Hadamard block <= 16384 (64 KiB of float32 in LDS)

int log2_block(int64_t len) {
  const int64_t b = len & -len;
  int lb = 0;
  while ((int64_t(1) << lb) < b) ++lb;
  return lb;
}

int cu_count() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
      cus = p.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return cus;
}

template <bool IB, bool OB, bool TR, int PT>
int launch_rht_vec_pt(const void *in, void *out, int64_t rows, int64_t n, int lb, const int8_t *signs,
                      float *rowsum, hipStream_t st) {
  const int64_t grid = rows < 8192 ? rows : 8192;
  const size_t shm = sizeof(float) * padded_floats((size_t)n);
  const int rc = allow_lds(rht_rows_vec<IB, OB, TR, PT>, shm + 1024);
  if (rc) return rc;
  hipLaunchKernelGGL((rht_rows_vec<IB, OB, TR, PT>), dim3((unsigned)grid), dim3(256), shm, st, in, out, rows, n,
                     lb, signs, rowsum);
  return hip_status(hipGetLastError());
}

// pieces of 8 per thread: n / 8 / 256 rounded up to a power of two
template <bool IB, bool OB, bool TR>
int launch_rht_vec(const void *in, void *out, int64_t rows, int64_t n, int lb, const int8_t *signs,
                   float *rowsum, hipStream_t st) {
  const int64_t pt = (n / 8 + 255) / 256;
  if (pt <= 1) return launch_rht_vec_pt<IB, OB, TR, 1>(in, out, rows, n, lb, signs, rowsum, st);
  if (pt <= 2) return launch_rht_vec_pt<IB, OB, TR, 2>(in, out, rows, n, lb, signs, rowsum, st);
  if (pt <= 4) return launch_rht_vec_pt<IB, OB, TR, 4>(in, out, rows, n, lb, signs, rowsum, st);
  if (pt <= 8) return launch_rht_vec_pt<IB, OB, TR, 8>(in, out, rows, n, lb, signs, rowsum, st);
  return launch_rht_vec_pt<IB, OB, TR, 16>(in, out, rows, n, lb, signs, rowsum, st);
}

// rows of n <= 4096 on 256-thread workgroups, longer rows on 512 or 1024
// threads (16 elements per thread)
template <bool IB, bool OB, bool TR, int NW, bool TILE16 = false>
int launch_rht_reg_nw(const void *in, void *out, int64_t rows, int64_t n, int lb, const int8_t *signs,
                      float *rowsum, hipStream_t st) {
  int64_t e = 1;
  while (e * 64 * NW < n) e <<= 1;
  const size_t shm = sizeof(float) * (size_t)(64 * NW * e + 64);
  // 1024 threads of 100+ registers each fill a CU: one resident workgroup per
  // CU, each streaming its rows with the next row's loads in flight (a second
  // round of workgroups measured 10% slower at 2048 x 16384)
  const int64_t cap = (int64_t)cu_count() * (NW == 16 ? 1 : 32 / NW);
  const int64_t grid = rows < cap ? rows : cap;
  const int rc = allow_lds(rht_rows_reg<IB, OB, TR, NW, TILE16>, shm + 64);
  if (rc) return rc;
  hipLaunchKernelGGL((rht_rows_reg<IB, OB, TR, NW, TILE16>), dim3((unsigned)grid), dim3(64 * NW), shm, st, in, out,
                     rows, (int)n, lb, signs, rowsum);
  return hip_status(hipGetLastError());
}

// rows of nb > 1 blocks of B = 1024, 2048 or 4096 (rht_rows_blk)
template <int NW, bool IB, bool OB, bool TR>
int launch_rht_blk_nw(const void *in, void *out, int64_t rows, int64_t n, const int8_t *signs, float *rowsum,
                      hipStream_t st) {
  constexpr int B = 1024 * NW;
  const int nb = (int)(n / B);
  const size_t shm = NW > 1 ? sizeof(float) * (size_t)nb * (B + 64) : 0;
  // about 24 waves a CU; a whole row of 16 waves (at most 64 VGPRs, 66 KiB of
  // LDS) gets two workgroups a CU, which keeps two rows in flight per CU
  // (2048 x 16384: 39 -> 34 us; wider grids measured no better elsewhere)
  const int wpc = nb * NW == 16 ? 32 : 24;
  const int64_t cap = (int64_t)cu_count() * (wpc / (nb * NW) > 1 ? wpc / (nb * NW) : 1);
  const int64_t grid = rows < cap ? rows : cap;
  const int rc = allow_lds(rht_rows_blk<NW, IB, OB, TR>, shm + 64);
  if (rc) return rc;
  hipLaunchKernelGGL((rht_rows_blk<NW, IB, OB, TR>), dim3((unsigned)grid), dim3(64 * NW * nb), shm, st, in, out, rows,
                     (int)n, nb, signs, rowsum);
  return hip_status(hipGetLastError());
}

template <bool IB, bool OB, bool TR>
int launch_rht_blk(const void *in, void *out, int64_t rows, int64_t n, int lb, const int8_t *signs, float *rowsum,
                   hipStream_t st) {
  switch (lb) {
    case 10: return launch_rht_blk_nw<1, IB, OB, TR>(in, out, rows, n, signs, rowsum, st);
    case 11: return launch_rht_blk_nw<2, IB, OB, TR>(in, out, rows, n, signs, rowsum, st);
    case 12: return launch_rht_blk_nw<4, IB, OB, TR>(in, out, rows, n, signs, rowsum, st);
    case 13: return launch_rht_blk_nw<8, IB, OB, TR>(in, out, rows, n, signs, rowsum, st);
    default: return launch_rht_blk_nw<16, IB, OB, TR>(in, out, rows, n, signs, rowsum, st);
  }
}

// x~ of at most 16 rows written in the small-batch GEMV's operand layout
// (tile16_index): bf16 in and out, n a multiple of 256 and at most 16384,
// 16-byte aligned pointers, in != out (rht_tile16_ok).
bool rht_tile16_ok(const void *in, const void *out, const int8_t *signs, int64_t rows, int64_t n) {
  return rows <= 16 && n % 256 == 0 && n <= 16384 && in != out &&
         ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(signs)) & 15) == 0;
}

int launch_rht_tile16(const void *in, void *out, int64_t rows, int64_t n, const int8_t *signs, float *rowsum,
                      hipStream_t st) {
  return launch_rht_reg_nw<true, true, false, 16, true>(in, out, rows, n, log2_block(n), signs, rowsum, st);
}

template <bool IB, bool OB, bool TR>
int launch_rht_reg(const void *in, void *out, int64_t rows, int64_t n, int lb, const int8_t *signs,
                   float *rowsum, hipStream_t st) {
  if (rows <= 64) return launch_rht_reg_nw<IB, OB, TR, 16>(in, out, rows, n, lb, signs, rowsum, st);
  if (n <= 4096) return launch_rht_reg_nw<IB, OB, TR, 4>(in, out, rows, n, lb, signs, rowsum, st);
  if (n <= 8192) return launch_rht_reg_nw<IB, OB, TR, 8>(in, out, rows, n, lb, signs, rowsum, st);
  return launch_rht_reg_nw<IB, OB, TR, 16>(in, out, rows, n, lb, signs, rowsum, st);
}

int launch_rht(const void *in, glq_dtype in_dt, void *out, glq_dtype out_dt, int64_t rows,
               int64_t n, const int8_t *signs, int transpose, float *rowsum, hipStream_t st) {
  const int lb = log2_block(n);
  if (lb > kMaxLogBlock) return GLQ_ERR_UNSUPPORTED;
  const bool aligned = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out) |
                         reinterpret_cast<uintptr_t>(signs)) & 15) == 0;
  // the block kernel for rows of whole blocks of 1024 .. 16384 (one
  // workgroup of at most 16 waves per row); the register kernel for a few
  // rows (decode-time batches, latency-bound: 1024 threads per row) and for
  // one-block rows the block kernel does not take; the LDS radix-16 kernel
  // for the remaining aligned rows
  const bool few = rows <= 64 && n % 8 == 0 && n <= 16384;
  // rows of whole blocks of 1024 .. 16384 (at most 16 waves a row): one
  // workgroup per row, the blocks' FWHTs in registers (rht_rows_blk)
  const int64_t nblk = n >> lb;
  if (lb >= 10 && lb <= 14 && (nblk << (lb - 10)) <= 16 && (nblk > 1 || !few) && aligned && in != out) {
    const bool ib = in_dt == GLQ_BF16, ob = out_dt == GLQ_BF16;
    if (transpose) {
      if (ib) return ob ? launch_rht_blk<true, true, true>(in, out, rows, n, lb, signs, rowsum, st)
                        : launch_rht_blk<true, false, true>(in, out, rows, n, lb, signs, rowsum, st);
      return ob ? launch_rht_blk<false, true, true>(in, out, rows, n, lb, signs, rowsum, st)
                : launch_rht_blk<false, false, true>(in, out, rows, n, lb, signs, rowsum, st);
    }
    if (ib) return ob ? launch_rht_blk<true, true, false>(in, out, rows, n, lb, signs, rowsum, st)
                      : launch_rht_blk<true, false, false>(in, out, rows, n, lb, signs, rowsum, st);
    return ob ? launch_rht_blk<false, true, false>(in, out, rows, n, lb, signs, rowsum, st)
              : launch_rht_blk<false, false, false>(in, out, rows, n, lb, signs, rowsum, st);
  }
  const bool one_block = n >= 1024 && n <= 16384 && (n & (n - 1)) == 0;
  if ((one_block || few) && aligned && in != out) {
    const bool ib = in_dt == GLQ_BF16, ob = out_dt == GLQ_BF16;
    if (transpose) {
      if (ib) return ob ? launch_rht_reg<true, true, true>(in, out, rows, n, lb, signs, rowsum, st)
                        : launch_rht_reg<true, false, true>(in, out, rows, n, lb, signs, rowsum, st);
      return ob ? launch_rht_reg<false, true, true>(in, out, rows, n, lb, signs, rowsum, st)
                : launch_rht_reg<false, false, true>(in, out, rows, n, lb, signs, rowsum, st);
    }
    if (ib) return ob ? launch_rht_reg<true, true, false>(in, out, rows, n, lb, signs, rowsum, st)
                      : launch_rht_reg<true, false, false>(in, out, rows, n, lb, signs, rowsum, st);
    return ob ? launch_rht_reg<false, true, false>(in, out, rows, n, lb, signs, rowsum, st)
              : launch_rht_reg<false, false, false>(in, out, rows, n, lb, signs, rowsum, st);
  }
  if (n % 8 == 0 && n <= RV_MAX && aligned && in != out) {
    const bool ib = in_dt == GLQ_BF16, ob = out_dt == GLQ_BF16;
    if (transpose) {
      if (ib) return ob ? launch_rht_vec<true, true, true>(in, out, rows, n, lb, signs, rowsum, st)
                        : launch_rht_vec<true, false, true>(in, out, rows, n, lb, signs, rowsum, st);
      return ob ? launch_rht_vec<false, true, true>(in, out, rows, n, lb, signs, rowsum, st)
                : launch_rht_vec<false, false, true>(in, out, rows, n, lb, signs, rowsum, st);
    }
    if (ib) return ob ? launch_rht_vec<true, true, false>(in, out, rows, n, lb, signs, rowsum, st)
                      : launch_rht_vec<true, false, false>(in, out, rows, n, lb, signs, rowsum, st);
    return ob ? launch_rht_vec<false, true, false>(in, out, rows, n, lb, signs, rowsum, st)
              : launch_rht_vec<false, false, false>(in, out, rows, n, lb, signs, rowsum, st);
  }
  // generic path: any n, in-place, unaligned pointers
  const int64_t grid = rows < 4096 ? rows : 4096;
  const size_t shm = sizeof(float) * padded_floats((size_t)1 << lb);
  const int rc = allow_lds(rht_rows, shm + 1024);
  if (rc) return rc;
  hipLaunchKernelGGL(rht_rows, dim3((unsigned)grid), dim3(256), shm, st, in, in_dt, out, out_dt,
                     rows, n, lb, signs, transpose, rowsum);
  return hip_status(hipGetLastError());
}

bool valid_dtype(int dt) { return dt == GLQ_F32 || dt == GLQ_BF16; }

int check_layer(const glq_layer *L, bool need_signs) {
  if (!L) return GLQ_ERR_ARG;
  if (L->n < 1 || L->k < 8 || L->k % 8 != 0) return GLQ_ERR_ARG;
  if (L->bpw != 2 && L->bpw != 3 && L->bpw != 4) return GLQ_ERR_ARG;
  if (L->bpw == 3 && L->resid_shift != 1) return GLQ_ERR_ARG;
  if (L->bpw == 4 && L->resid_shift != 2) return GLQ_ERR_ARG;
  if (!(std::isfinite(L->scale) && L->scale > 0.0f)) return GLQ_ERR_ARG;
  if (!L->idx1 || !L->cb) return GLQ_ERR_ARG;
  if (L->bpw > 2 && !L->idx2) return GLQ_ERR_ARG;
  if (need_signs && (!L->sign_k || !L->sign_n)) return GLQ_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(L->row_scale) & 3) return GLQ_ERR_ARG;
  if ((double)L->n * (double)L->k > 17179869184.0) return GLQ_ERR_UNSUPPORTED;
  return GLQ_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The decode-GEMM's k split (gemm8_bf16<., ., true>): used when a layer has
// fewer 256 x 256 tiles than CUs and long rows (remainders of at least 32
// k-steps). The E = CUs - tiles
// free CUs run q = ceil(tiles / E) remainders each (at most 4), so a
// remainder of r = (S - 2 q) / (q + 1) steps balances a main part's S - r
// against q (r + 2); s_main = S - r is made even (the x~ double buffer starts
// on its first half).
struct G8Plan { bool split = false; int64_t s_main = 0; int64_t grid = 0; };

G8Plan g8_plan(int64_t m, int64_t n, int64_t k) {
  G8Plan pl;
  if (m <= 16 || k % GM_BK != 0) return pl;
  const int64_t tiles = ((m + GM_BM - 1) / GM_BM) * ((n + GM_BN - 1) / GM_BN);
  const int64_t S = k / GM_BK, cus = cu_count();
  if (tiles >= cus || S < 64 || tiles >= 1008) return pl;
  const int64_t extra = cus - tiles;
  const int64_t q = (tiles + extra - 1) / extra;
  if (q > 4) return pl;
  // each remainder also pays about two k-steps of fixed cost (its table
  // copy, prologue and partial sums), which the q in a row on one CU add up
  int64_t r = (S - 2 * q) / (q + 1);
  if ((S - r) % 2) ++r;
  // a remainder pays the table copy, its prologue and the partial sums: below
  // 32 k-steps that outweighs the CUs it brings (3072^2 at 4,096 tokens, 12
  // steps: 87 -> 104 us; the 3072 x 12288 down projection, 48: 334 -> 315 us)
  if (r < 32 || S - r < 2) return pl;
  pl.split = true;
  pl.s_main = S - r;
  pl.grid = 2 * tiles;
  return pl;
}

// Workspace: control words (GLQ_WS_CTRL_BYTES; the single-launch layer's
// counters and the k split's tile counters: zero before first use, left zero
// by every call), then x~, row sums of x~, z = s W^ x~, and the k split's
// float32 partial sums (two 256 KiB halves per tile, only for layers the
// split applies to).
struct WsLayout { size_t ctrl, xt, rowsum, z, part, total; };

WsLayout ws_layout(int64_t n, int64_t k, int64_t m) {
  WsLayout w;
  w.ctrl = 0;
  w.xt = kCtrlBytes;
  // x~: float32 [m][k], or bf16 in the 16-row operand layout when m <= 16
  const size_t xt_bytes = (size_t)(m <= 16 ? 16 : m) * (size_t)k * 4;
  w.rowsum = w.xt + align256(xt_bytes);
  w.z = w.rowsum + align256((size_t)m * 4);
  w.part = w.z + align256((size_t)m * (size_t)n * 4);
  const G8Plan pl = g8_plan(m, n, k);
  const int64_t tiles = ((m + GM_BM - 1) / GM_BM) * ((n + GM_BN - 1) / GM_BN);
  w.total = w.part + (pl.split ? (size_t)tiles * 2 * 65536 * 4 : 0);
  return w;
}

template <int BPW>
int launch_decode(const glq_layer *L, void *w_out, glq_dtype out_dt, hipStream_t st) {
  const int64_t groups = L->n * (L->k / 8);
  const size_t shm = lds_table_bytes<BPW>();
  int64_t grid = (groups + 255) / 256;
  const int64_t cap = (int64_t)cu_count() * 4;
  if (grid > cap) grid = cap;
  const uint8_t *blob = reinterpret_cast<const uint8_t *>(L->cb);
  int rc = out_dt == GLQ_F32 ? allow_lds(decode_weights_k<BPW, true>, shm)
                             : allow_lds(decode_weights_k<BPW, false>, shm);
  if (rc) return rc;
  if (out_dt == GLQ_F32)
    hipLaunchKernelGGL((decode_weights_k<BPW, true>), dim3((unsigned)grid), dim3(256), shm, st,
                       L->idx1, L->idx2, blob, L->scale, L->row_scale, (uint32_t)(L->k / 8), groups, w_out);
  else
    hipLaunchKernelGGL((decode_weights_k<BPW, false>), dim3((unsigned)grid), dim3(256), shm, st,
                       L->idx1, L->idx2, blob, L->scale, L->row_scale, (uint32_t)(L->k / 8), groups, w_out);
  return hip_status(hipGetLastError());
}

// Row tiles per GEMV workgroup: more than one only where it measured faster
// (2 bpw layers of at least 1024 tiles, e.g. 16384 x 16384: 60 -> 41 us at
// m = 8); at 3/4 bpw the extra accumulators spill.
int gv_row_tiles(int bpw, int64_t tiles) { return bpw == 2 && tiles >= 1024 ? 4 : 1; }

template <int BPW>
int launch_matmul(const glq_layer *L, const void *xt, glq_dtype x_dt, const float *rowsum, int64_t m,
                  void *out, glq_dtype out_dt, hipStream_t st, bool tiled = false, unsigned int *ctrl = nullptr,
                  float *part = nullptr) {
  const uint8_t *blob = reinterpret_cast<const uint8_t *>(L->cb);
  const size_t tab = lds_table_bytes<BPW>();
  if (x_dt == GLQ_F32) {
    int rc0 = allow_lds(gemv_f32<BPW>, tab);
    if (rc0) return rc0;
    int64_t grid = (L->n + 3) / 4;
    const int64_t cap = (int64_t)cu_count() * 8;
    if (grid > cap) grid = cap;
    for (int64_t m0 = 0; m0 < m; m0 += 4) {
      const int64_t mc = m - m0 < 4 ? m - m0 : 4;
      hipLaunchKernelGGL(gemv_f32<BPW>, dim3((unsigned)grid), dim3(256), tab, st, L->idx1, L->idx2,
                         blob, reinterpret_cast<const float *>(xt), m0, mc, L->n, L->k, L->scale, L->row_scale,
                         out, out_dt);
      int rc = hip_status(hipGetLastError());
      if (rc) return rc;
    }
    return GLQ_OK;
  }
  const float post = L->scale * Epi<BPW>::mul;
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(xt);
  if (m <= 16) {
    // row tiles per workgroup: each x~ operand load serves 16 RT weight rows;
    // keep at least ~128 workgroups in flight
    const int64_t tiles = (L->n + 15) / 16;
    const int rt = gv_row_tiles(BPW, tiles);
    const int64_t grid = (tiles + rt - 1) / rt;
    const size_t shm = tab + (size_t)rt * GV_WAVES * 16 * 16 * 4;
    const bool g8 = ((L->k / 8) % 8) == 0;
    constexpr int RT4 = BPW == 2 ? 4 : 1;            // the only multi-tile variant
    auto kern = tiled ? (rt == 4 ? gemv_bf16<BPW, true, RT4, true> : gemv_bf16<BPW, true, 1, true>)
              : g8 ? (rt == 4 ? gemv_bf16<BPW, true, RT4, false> : gemv_bf16<BPW, true, 1, false>)
                   : (rt == 4 ? gemv_bf16<BPW, false, RT4, false> : gemv_bf16<BPW, false, 1, false>);
    int rc = allow_lds(kern, shm);
    if (rc) return rc;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * GV_WAVES), shm, st, L->idx1, L->idx2, blob, xb,
                       rowsum, m, L->n, L->k, post, L->row_scale, out, out_dt);
  } else {
    const int64_t mb = (m + GM_BM - 1) / GM_BM, nb = (L->n + GM_BN - 1) / GM_BN;
    const int64_t tiles = mb * nb;
    if (tiles > 0x7FFFFFFF) return GLQ_ERR_UNSUPPORTED;
    const size_t shm = tab + 2 * GM_A_BYTES;       // >= G8_EPI_BYTES: the 8-wave epilogue fits
    const bool even_g = ((L->k / 8) % 4) == 0;
    // gemm8_bf16: whole x~ tiles and 32-bit buffer offsets (256 rows of x~)
    const bool k64 = L->k % GM_BK == 0 && (int64_t)GM_BM * L->k * 2 < 0x7FFFFFFF;
    const bool ob = out_dt == GLQ_BF16;
    const int vec = ((L->n * (ob ? 2 : 4)) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) ? 1 : 0;
    if (k64) {
      const G8Plan pl = part && ctrl ? g8_plan(m, L->n, L->k) : G8Plan{};
      G8Split sp{part, ctrl, pl.s_main};
      auto kern = pl.split ? (ob ? gemm8_bf16<BPW, true, true> : gemm8_bf16<BPW, false, true>)
                           : (ob ? gemm8_bf16<BPW, true, false> : gemm8_bf16<BPW, false, false>);
      int rc = allow_lds(kern, shm);
      if (rc) return rc;
      hipLaunchKernelGGL(kern, dim3((unsigned)(pl.split ? pl.grid : tiles)), dim3(G8_THREADS), shm, st, L->idx1,
                         L->idx2, blob, xb, rowsum, m, L->n, L->k, post, L->row_scale, out, vec, mb, tiles, sp);
    } else {
      auto kern = even_g ? (ob ? gemm_bf16<BPW, true, true> : gemm_bf16<BPW, true, false>)
                         : (ob ? gemm_bf16<BPW, false, true> : gemm_bf16<BPW, false, false>);
      int rc = allow_lds(kern, shm);
      if (rc) return rc;
      hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), shm, st, L->idx1, L->idx2, blob, xb, rowsum, m,
                         L->n, L->k, post, L->row_scale, out, vec, mb, tiles);
    }
  }
  return hip_status(hipGetLastError());
}

}  // namespace
}  // namespace glq

// ---------------------------------------------------------------- static scratch
// The workspace of glq_fused_linear_noalloc: one array per GPU, created with
// the code object and held until the process ends. Host code never takes
// this name as an address (on the host it is only a stand-in for the
// symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[GLQ_STATIC_WS_BYTES];

namespace glq {
namespace {

__global__ void __launch_bounds__(256) zero_words(uint32_t *p, uint32_t count) {
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < count; i += gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct StaticWs {
  std::once_flag once;
  uint8_t *ptr = nullptr;                 // device address of this GPU's scratch
  int rc = GLQ_OK;
  std::atomic<bool> dirty{true};          // control words to clear before the next use
};
StaticWs g_static_ws[kMaxDevices];

// The current device's scratch, its address looked up on the first call on
// that device; its control words are cleared (a fill kernel on the caller's
// stream, ordered before the layer's kernels) on first use and after a call
// that failed in HIP.
int static_workspace(hipStream_t st, uint8_t **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_last_error, sizeof g_last_error, "glq_fused_linear_noalloc: device %d beyond %d", dev, kMaxDevices);
    return GLQ_ERR_UNSUPPORTED;
  }
  StaticWs &w = g_static_ws[dev];
  std::call_once(w.once, [&] {
    void *p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p) {
      w.rc = err != hipSuccess ? hip_status(err, "hipGetSymbolAddress(scratch)") : GLQ_ERR_HIP;
      return;
    }
    w.ptr = reinterpret_cast<uint8_t *>(p);
  });
  if (w.rc) return w.rc;
  if (w.dirty.exchange(false)) {
    hipLaunchKernelGGL(zero_words, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t *>(w.ptr),
                       (uint32_t)(kCtrlBytes / 4));
    const int rc = hip_status(hipGetLastError(), "zero_words");
    if (rc) {
      w.dirty = true;
      return rc;
    }
  }
  *out = w.ptr;
  return GLQ_OK;
}

void static_workspace_failed() {
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) g_static_ws[dev].dirty = true;
}

}  // namespace
}  // namespace glq

using namespace glq;

extern "C" int glq_rht_apply(const void *in, glq_dtype in_dt, void *out, glq_dtype out_dt,
                             int64_t rows, int64_t n, const int8_t *signs, int32_t transpose,
                             void *hip_stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(out_dt)) return GLQ_ERR_ARG;
  if (rows < 0 || n < 1 || (transpose != 0 && transpose != 1)) return GLQ_ERR_ARG;
  if (rows == 0) return GLQ_OK;
  if (!in || !out || !signs) return GLQ_ERR_ARG;
  if (in == out && in_dt != out_dt) return GLQ_ERR_ARG;
  return launch_rht(in, in_dt, out, out_dt, rows, n, signs, transpose, nullptr,
                    reinterpret_cast<hipStream_t>(hip_stream));
}

extern "C" int glq_decode_weights(const glq_layer *L, void *w_out, glq_dtype out_dt, void *hip_stream) {
  int rc = check_layer(L, false);
  if (rc) return rc;
  if (!w_out || !valid_dtype(out_dt)) return GLQ_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  switch (L->bpw) {
    case 2: return launch_decode<2>(L, w_out, out_dt, st);
    case 3: return launch_decode<3>(L, w_out, out_dt, st);
    default: return launch_decode<4>(L, w_out, out_dt, st);
  }
}

extern "C" const char *glq_last_error(void) { return g_last_error; }

extern "C" size_t glq_fused_linear_workspace(const glq_layer *L, int64_t m) {
  if (!L || m <= 0 || L->n < 1 || L->k < 8) return 0;
  return ws_layout(L->n, L->k, m).total;
}

extern "C" int glq_fused_linear(const glq_layer *L, const void *x, glq_dtype x_dt, int64_t m, void *y,
                                glq_dtype y_dt, void *workspace, size_t ws_bytes, uint32_t flags,
                                void *hip_stream) {
  const bool in_rht = !(flags & GLQ_FLAG_NO_INPUT_RHT);
  const bool out_rht = !(flags & GLQ_FLAG_NO_OUTPUT_RHT);
  int rc = check_layer(L, in_rht || out_rht);
  if (rc) return rc;
  if (flags & ~3u) return GLQ_ERR_ARG;
  if (!valid_dtype(x_dt) || !valid_dtype(y_dt) || m < 0) return GLQ_ERR_ARG;
  if (m == 0) return GLQ_OK;
  if (!x || !y) return GLQ_ERR_ARG;
  const WsLayout ws = ws_layout(L->n, L->k, m);
  if (!workspace || ws_bytes < ws.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return GLQ_ERR_WORKSPACE;
  if (!in_rht && (reinterpret_cast<uintptr_t>(x) & 15)) return GLQ_ERR_ARG;   // loaded 16 B at a time
  if (in_rht && log2_block(L->k) > kMaxLogBlock) return GLQ_ERR_UNSUPPORTED;
  if (out_rht && log2_block(L->n) > kMaxLogBlock) return GLQ_ERR_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  uint8_t *wsb = reinterpret_cast<uint8_t *>(workspace);
  void *xt = wsb + ws.xt;
  float *rowsum = reinterpret_cast<float *>(wsb + ws.rowsum);
  float *z = reinterpret_cast<float *>(wsb + ws.z);
  unsigned int *ctrl_w = reinterpret_cast<unsigned int *>(wsb + ws.ctrl);
  float *part = ws.total > ws.part ? reinterpret_cast<float *>(wsb + ws.part) : nullptr;

  // whole layer in one launch at decode-time batch sizes
  if (x_dt == GLQ_BF16 && in_rht && out_rht && m <= 4 && m * L->k <= LY_MAXE && m * L->n <= LY_MAXE &&
      (L->k / 8) % 8 == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(L->idx1)) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(L->sign_k) & 7) == 0 &&
      (L->bpw != 4 || (reinterpret_cast<uintptr_t>(L->idx2) & 15) == 0) &&
      (L->bpw != 3 || (reinterpret_cast<uintptr_t>(L->idx2) & 7) == 0)) {
    const int64_t tiles = (L->n + 15) / 16;
    const int64_t grid = tiles < cu_count() ? tiles : cu_count();
    const float post = L->scale * (L->bpw == 2 ? 1.0f : L->bpw == 3 ? 0.25f : 0.125f);
    unsigned int *counter = reinterpret_cast<unsigned int *>(wsb + ws.ctrl);
    const uint8_t *blob = reinterpret_cast<const uint8_t *>(L->cb);
    const uint16_t *xb = reinterpret_cast<const uint16_t *>(x);
    const int lbk = log2_block(L->k), lbn = log2_block(L->n);
#define GLQ_LAYER_SMALL(B)                                                                              \
  do {                                                                                                  \
    rc = allow_lds(layer_small<B>, ly_lds_bytes<B>());                                                  \
    if (rc) return rc;                                                                                  \
    hipLaunchKernelGGL(layer_small<B>, dim3((unsigned)grid), dim3(64 * GV_WAVES), ly_lds_bytes<B>(), st, \
                       L->idx1, L->idx2, blob, xb, L->sign_k, L->sign_n, m, L->n, L->k, lbk, lbn, post,   \
                       L->row_scale, y, y_dt, z, counter);                                                               \
  } while (0)
    if (L->bpw == 2) GLQ_LAYER_SMALL(2);
    else if (L->bpw == 3) GLQ_LAYER_SMALL(3);
    else GLQ_LAYER_SMALL(4);
#undef GLQ_LAYER_SMALL
    return hip_status(hipGetLastError());
  }
  const void *xt_use = x;
  bool tiled = false;
  if (x_dt == GLQ_F32) {
    if (in_rht) {
      rc = launch_rht(x, GLQ_F32, xt, GLQ_F32, m, L->k, L->sign_k, 0, nullptr, st);
      if (rc) return rc;
      xt_use = xt;
    }
  } else {
    if (in_rht && rht_tile16_ok(x, xt, L->sign_k, m, L->k)) {
      // at most 16 rows: x~ straight into the GEMV's operand layout
      rc = launch_rht_tile16(x, xt, m, L->k, L->sign_k, rowsum, st);
      if (rc) return rc;
      xt_use = xt;
      tiled = true;
    } else if (in_rht) {
      rc = launch_rht(x, GLQ_BF16, xt, GLQ_BF16, m, L->k, L->sign_k, 0, rowsum, st);
      if (rc) return rc;
      xt_use = xt;
    } else if (L->bpw > 2) {
      const int64_t grid = m < 4096 ? m : 4096;
      hipLaunchKernelGGL(row_sums_bf16, dim3((unsigned)grid), dim3(256), 0, st,
                         reinterpret_cast<const uint16_t *>(x), m, L->k, rowsum);
      rc = hip_status(hipGetLastError());
      if (rc) return rc;
    }
  }
  // z between the matrix product and the output rotation: float32, except on
  // the prefill path with a bf16 y, where it is rounded to bf16 (half the
  // bytes of the largest intermediate; the extra rounding is a relative
  // 2^-9 per element of z, spread over the Hadamard sums)
  void *mm_out = out_rht ? (void *)z : y;
  const glq_dtype mm_dt = !out_rht ? y_dt : (x_dt == GLQ_BF16 && y_dt == GLQ_BF16 && m > 16) ? GLQ_BF16 : GLQ_F32;
  switch (L->bpw) {
    case 2: rc = launch_matmul<2>(L, xt_use, x_dt, rowsum, m, mm_out, mm_dt, st, tiled, ctrl_w, part); break;
    case 3: rc = launch_matmul<3>(L, xt_use, x_dt, rowsum, m, mm_out, mm_dt, st, tiled, ctrl_w, part); break;
    default: rc = launch_matmul<4>(L, xt_use, x_dt, rowsum, m, mm_out, mm_dt, st, tiled, ctrl_w, part); break;
  }
  if (rc) return rc;
  if (out_rht) return launch_rht(z, mm_dt, y, y_dt, m, L->n, L->sign_n, 1, nullptr, st);
  return GLQ_OK;
}

extern "C" int glq_fused_linear_noalloc(const glq_layer *L, const void *x, glq_dtype x_dt, int64_t m, void *y,
                                        glq_dtype y_dt, uint32_t flags, void *hip_stream) {
  const bool in_rht = !(flags & GLQ_FLAG_NO_INPUT_RHT);
  const bool out_rht = !(flags & GLQ_FLAG_NO_OUTPUT_RHT);
  int rc = check_layer(L, in_rht || out_rht);
  if (rc) return rc;
  if (m < 0) return GLQ_ERR_ARG;
  if (m == 0) return GLQ_OK;
  const size_t need = ws_layout(L->n, L->k, m).total;
  if (need > (size_t)GLQ_STATIC_WS_BYTES) {
    snprintf(g_last_error, sizeof g_last_error,
             "glq_fused_linear_noalloc: %zu bytes of workspace needed, the static scratch holds %zu",
             need, (size_t)GLQ_STATIC_WS_BYTES);
    return GLQ_ERR_WORKSPACE;
  }
  uint8_t *ws = nullptr;
  rc = static_workspace(reinterpret_cast<hipStream_t>(hip_stream), &ws);
  if (rc) return rc;
  rc = glq_fused_linear(L, x, x_dt, m, y, y_dt, ws, (size_t)GLQ_STATIC_WS_BYTES, flags, hip_stream);
  if (rc == GLQ_ERR_HIP) static_workspace_failed();
  return rc;
}

extern "C" int glq_ep_decode_weights(const glq_ep_layer *L, void *w_out, glq_dtype out_dt, void *hip_stream) {
  if (!L || !w_out || !valid_dtype(out_dt)) return GLQ_ERR_ARG;
  if (L->n < 1 || L->k < 8 || L->k % 8 != 0 || L->lane_groups < 1 || L->lane_groups > (1 << 20)) return GLQ_ERR_ARG;
  if (!(L->step > 0.0f) || !std::isfinite(L->step)) return GLQ_ERR_ARG;
  if (!L->row_scale || !L->states || !L->offsets || !L->lut) return GLQ_ERR_ARG;
  if (L->nwords < 0 || L->nwords > 0xFFFFFFF0ll || !L->words) return GLQ_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(w_out) & 15) || (reinterpret_cast<uintptr_t>(L->lut) & 15) ||
      (reinterpret_cast<uintptr_t>(L->words) & 15))
    return GLQ_ERR_ARG;
  if ((double)L->n * (double)L->k / 8.0 >= 2147483648.0) return GLQ_ERR_UNSUPPORTED;
  const uint32_t total = (uint32_t)(L->n * (L->k / 8));
  const uint64_t bg = 64ull * (uint64_t)L->lane_groups;
  const uint32_t nblocks = (uint32_t)((total + bg - 1) / bg);
  // one wave per block: 4-wave workgroups spread a layer of at most one
  // wave per SIMD over every CU; larger layers take 8 (two per CU fit)
  const bool wide = nblocks > (uint32_t)cu_count() * 4;
  const uint32_t waves = wide ? 8 : 4;
  const uint32_t grid = (nblocks + waves - 1) / waves;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  auto kern = wide ? (out_dt == GLQ_F32 ? ep_decode_k<true, 8> : ep_decode_k<false, 8>)
                   : (out_dt == GLQ_F32 ? ep_decode_k<true, 4> : ep_decode_k<false, 4>);
  int rc = allow_lds(kern, ep_lds(waves));
  if (rc) return rc;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), ep_lds(waves), st, L->states, L->offsets, L->words,
                     (uint32_t)L->nwords, reinterpret_cast<const uint8_t *>(L->lut), L->row_scale, L->step, total,
                     (uint32_t)(L->k / 8), (uint32_t)L->lane_groups, nblocks, (uint32_t)L->k, w_out);
  return hip_status(hipGetLastError());
}

int launch_gemm_w(const uint16_t *w, const uint16_t *xt, int64_t m, int64_t n, int64_t k, void *out,
                  glq_dtype out_dt, hipStream_t st) {
  if (m <= 16) {
    const int64_t grid = (n + 15) / 16;
    if (grid > 0x7FFFFFFF) return GLQ_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(gemv_w_bf16, dim3((unsigned)grid), dim3(64 * GW_WAVES), 0, st, w, xt, m, n, k, 1.0f, out,
                       out_dt);
    return hip_status(hipGetLastError());
  }
  const int64_t mb = (m + GM_BM - 1) / GM_BM, nb = (n + GM_BN - 1) / GM_BN;
  const int64_t tiles = mb * nb;
  if (tiles > 0x7FFFFFFF) return GLQ_ERR_UNSUPPORTED;
  // k a multiple of 64: gemm_w2_bf16; otherwise gemm_w_bf16_lds (4 waves of
  // 64 weight rows, pointer loads, partial last tile)
  const bool direct = k % GM_BK == 0;
  const size_t shm = 4 * GM_A_BYTES;
  const bool ob = out_dt == GLQ_BF16;
  const int vec = ((n * (ob ? 2 : 4)) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) ? 1 : 0;
  if (direct && (int64_t)GM_BM * k * 2 < 0x7FFFFFFF) {
    // 2 x 2 wave tiles, both operands through LDS (buffer loads, 32-bit offsets)
    auto k2 = ob ? gemm_w2_bf16<true> : gemm_w2_bf16<false>;
    const size_t shm2 = 4 * GM_A_BYTES;
    int rc = allow_lds(k2, shm2);
    if (rc) return rc;
    hipLaunchKernelGGL(k2, dim3((unsigned)tiles), dim3(256), shm2, st, w, xt, m, n, k, 1.0f, out, vec, mb, tiles);
    return hip_status(hipGetLastError());
  }
  auto kern = ob ? gemm_w_bf16_lds<true> : gemm_w_bf16_lds<false>;
  int rc = allow_lds(kern, shm);
  if (rc) return rc;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), shm, st, w, xt, m, n, k, 1.0f, out, vec, mb, tiles);
  return hip_status(hipGetLastError());
}

// LDS bytes of ep_gemv_k for this layer at `waves` waves per workgroup, or 0
// where the fused batch-1 product does not apply: m != 1, k / 8 < 64 (a block
// of groups would span too many rows for the LDS row sums), or a layer of
// 2^31 groups or more.
size_t ep_gemv_shm(const glq_ep_layer *L, int64_t m, uint32_t waves) {
  if (m != 1 || L->k < 512 || L->k % 8 != 0 || L->n < 1 || L->lane_groups < 1 || L->lane_groups > (1 << 20))
    return 0;
  if ((double)L->n * (double)L->k / 8.0 >= 2147483648.0) return 0;
  const uint64_t gpr = (uint64_t)(L->k / 8), bg = 64ull * (uint64_t)L->lane_groups;
  const uint64_t rmax = (bg + gpr - 2) / gpr + 1;      // rows a block of bg groups can touch
  const uint64_t shm = ep_lds(waves) + (uint64_t)waves * rmax * 4;
  return shm <= 160 * 1024 ? (size_t)shm : 0;
}

__global__ void __launch_bounds__(256) f32_to_bf16_k(const float *__restrict__ in, uint16_t *__restrict__ out,
                                                     uint32_t count) {
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < count; i += gridDim.x * 256)
    out[i] = f32_to_bf16_rne(in[i]);
}

// The batch-1 product fused with the decode (ep_gemv_shm(L, m, 8) != 0): x~
// (bf16) from the input transform (or x itself), z zeroed, then ep_gemv_k
// summing into z (float32 [n]).
int launch_ep_gemv(const glq_ep_layer *L, const void *x, glq_dtype x_dt, bool in_rht, int64_t m, uint16_t *xt,
                   float *z, hipStream_t st) {
  if (!(L->step > 0.0f) || !std::isfinite(L->step)) return GLQ_ERR_ARG;
  if (!L->row_scale || !L->states || !L->offsets || !L->lut) return GLQ_ERR_ARG;
  if (L->nwords < 0 || L->nwords > 0xFFFFFFF0ll || !L->words) return GLQ_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(L->lut) & 15) || (reinterpret_cast<uintptr_t>(L->words) & 15)) return GLQ_ERR_ARG;
  const uint32_t gpr = (uint32_t)(L->k / 8);
  const uint32_t total = (uint32_t)(L->n * gpr);
  const uint64_t bg = 64ull * (uint64_t)L->lane_groups;
  const uint32_t nblocks = (uint32_t)((total + bg - 1) / bg);
  const uint32_t rmax = (uint32_t)((bg + gpr - 2) / gpr + 1);
  // as in the decode: 4-wave workgroups while one wave per SIMD covers the
  // layer, 8 beyond
  const bool wide = nblocks > (uint32_t)cu_count() * 4;
  const uint32_t waves = wide ? 8 : 4;
  const size_t shm = ep_gemv_shm(L, m, waves);
  if (!shm) return GLQ_ERR_UNSUPPORTED;
  const uint16_t *xt_use = reinterpret_cast<const uint16_t *>(x);
  int rc;
  if (in_rht) {
    rc = launch_rht(x, x_dt, xt, GLQ_BF16, m, L->k, L->sign_k, 0, nullptr, st);
    if (rc) return rc;
    xt_use = xt;
  }
  const uint32_t zw = (uint32_t)(m * L->n);
  hipLaunchKernelGGL(zero_words, dim3((zw + 255) / 256 < 1024 ? (zw + 255) / 256 : 1024), dim3(256), 0, st,
                     reinterpret_cast<uint32_t *>(z), zw);
  rc = hip_status(hipGetLastError(), "zero_words");
  if (rc) return rc;
  const uint32_t grid = (nblocks + waves - 1) / waves;
  auto kern = wide ? ep_gemv_k<8> : ep_gemv_k<4>;
  rc = allow_lds(kern, shm);
  if (rc) return rc;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), shm, st, L->states, L->offsets, L->words, (uint32_t)L->nwords,
                     reinterpret_cast<const uint8_t *>(L->lut), L->row_scale, L->step, total, gpr,
                     (uint32_t)L->lane_groups, nblocks, xt_use, z, rmax);
  return hip_status(hipGetLastError(), "ep_gemv_k");
}

// Workspace of the entropy-coded layer: decoded W^ (bf16; absent where the
// fused batch-1 product applies), x~ (bf16), z (float32).
struct EpWs { size_t w, xt, z, total; };
EpWs ep_ws_layout(const glq_ep_layer *L, int64_t m) {
  const int64_t n = L->n, k = L->k;
  EpWs e;
  e.w = 0;
  e.xt = ep_gemv_shm(L, m, 8) ? 0 : align256((size_t)n * (size_t)k * 2);
  e.z = e.xt + align256((size_t)m * (size_t)k * 2);
  e.total = e.z + align256((size_t)m * (size_t)n * 4);
  return e;
}

extern "C" size_t glq_ep_fused_linear_workspace(const glq_ep_layer *L, int64_t m) {
  if (!L || m <= 0 || L->n < 1 || L->k < 8) return 0;
  return ep_ws_layout(L, m).total;
}

extern "C" int glq_ep_fused_linear(const glq_ep_layer *L, const void *x, glq_dtype x_dt, int64_t m, void *y,
                                   glq_dtype y_dt, void *workspace, size_t ws_bytes, uint32_t flags,
                                   void *hip_stream) {
  const bool in_rht = !(flags & GLQ_FLAG_NO_INPUT_RHT);
  const bool out_rht = !(flags & GLQ_FLAG_NO_OUTPUT_RHT);
  if (!L || (flags & ~3u) || !valid_dtype(x_dt) || !valid_dtype(y_dt) || m < 0) return GLQ_ERR_ARG;
  if ((in_rht && !L->sign_k) || (out_rht && !L->sign_n)) return GLQ_ERR_ARG;
  if (m == 0) return GLQ_OK;
  if (!x || !y) return GLQ_ERR_ARG;
  if (!in_rht && (x_dt != GLQ_BF16 || (reinterpret_cast<uintptr_t>(x) & 15))) return GLQ_ERR_UNSUPPORTED;
  if (in_rht && log2_block(L->k) > kMaxLogBlock) return GLQ_ERR_UNSUPPORTED;
  if (out_rht && log2_block(L->n) > kMaxLogBlock) return GLQ_ERR_UNSUPPORTED;
  if (L->n < 1 || L->k < 8 || L->k % 8 != 0) return GLQ_ERR_ARG;
  const EpWs ws = ep_ws_layout(L, m);
  if (!workspace || ws_bytes < ws.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) return GLQ_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  uint8_t *wsb = reinterpret_cast<uint8_t *>(workspace);
  uint16_t *w = reinterpret_cast<uint16_t *>(wsb + ws.w);
  uint16_t *xt = reinterpret_cast<uint16_t *>(wsb + ws.xt);
  void *z = wsb + ws.z;
  int rc;
  if (ep_gemv_shm(L, m, 8)) {
    // batch 1: the decode fused into the product (ep_gemv_k), summed in
    // float32 into z, or straight into a float32 y without the output transform
    const bool direct = !out_rht && y_dt == GLQ_F32 && !(reinterpret_cast<uintptr_t>(y) & 3);
    rc = launch_ep_gemv(L, x, x_dt, in_rht, m, xt, reinterpret_cast<float *>(direct ? y : z), st);
    if (rc || direct) return rc;
    if (out_rht) return launch_rht(z, GLQ_F32, y, y_dt, m, L->n, L->sign_n, 1, nullptr, st);
    const uint32_t cnt = (uint32_t)(m * L->n);
    hipLaunchKernelGGL(f32_to_bf16_k, dim3((cnt + 255) / 256 < 1024 ? (cnt + 255) / 256 : 1024), dim3(256), 0, st,
                       reinterpret_cast<const float *>(z), reinterpret_cast<uint16_t *>(y), cnt);
    return hip_status(hipGetLastError(), "f32_to_bf16_k");
  }
  rc = glq_ep_decode_weights(L, w, GLQ_BF16, hip_stream);
  if (rc) return rc;
  const uint16_t *xt_use = reinterpret_cast<const uint16_t *>(x);
  if (in_rht) {
    rc = launch_rht(x, x_dt, xt, GLQ_BF16, m, L->k, L->sign_k, 0, nullptr, st);
    if (rc) return rc;
    xt_use = xt;
  }
  void *mm_out = out_rht ? z : y;
  const glq_dtype mm_dt = !out_rht ? y_dt : (y_dt == GLQ_BF16 && m > 16) ? GLQ_BF16 : GLQ_F32;
  rc = launch_gemm_w(w, xt_use, m, L->n, L->k, mm_out, mm_dt, st);
  if (rc) return rc;
  if (out_rht) return launch_rht(z, mm_dt, y, y_dt, m, L->n, L->sign_n, 1, nullptr, st);
  return GLQ_OK;
}
