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
//   decode_weights  indices -> W^ (rotated basis) as float32 or bf16.
//   gemv_bf16       m <= 16: one 16-row weight tile per workgroup, 4 waves split
//                   k, bf16 MFMA 16x16x32 with x~ rows as the M side (the few
//                   activation rows are padded to 16) and weights decoded
//                   straight into the B operand registers.
//   gemm_bf16       m > 16: 128 x 128 output tiles, x~ staged through LDS,
//                   weights decoded per wave straight into MFMA B operands.
//   gemv_f32        float32 path: exact float32 weights, float32 FMAs.
//
// Every kernel that decodes first copies the decode tables (glq_tables.h) from
// the caller's GLQ_CB_DEVICE buffer into LDS.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "glq.h"
#include "glq_tables.h"

namespace glq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- LDS tables
// LDS layout of the decode tables: [CT][OT][HT stage 1][HT stage 2 | R3]
constexpr uint32_t kLdsCt = 0;
constexpr uint32_t kLdsOt = kLdsCt + kCtBytes;
constexpr uint32_t kLdsHt1 = kLdsOt + kOtBytes;
constexpr uint32_t kLdsHt2 = kLdsHt1 + kHtBytes;

template <int BPW> struct TabCfg;
template <> struct TabCfg<2> { static constexpr uint32_t ht1 = kHtBf16Off, ht2 = 0, ht2_bytes = 0; };
template <> struct TabCfg<3> { static constexpr uint32_t ht1 = kHtA3Off, ht2 = kR3Off, ht2_bytes = kR3Bytes; };
template <> struct TabCfg<4> { static constexpr uint32_t ht1 = kHtA4Off, ht2 = kHtB4Off, ht2_bytes = kHtBytes; };

template <int BPW>
constexpr uint32_t lds_table_bytes() { return kLdsHt2 + TabCfg<BPW>::ht2_bytes; }

// Copy CT + OT + the two value tables of this bit width into LDS.
template <int BPW>
__device__ __forceinline__ void load_tables(uint8_t *lds, const uint8_t *blob) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  // CT and OT are contiguous in the blob and in LDS
  const uint4 *src0 = reinterpret_cast<const uint4 *>(blob + kCtOff);
  uint4 *dst0 = reinterpret_cast<uint4 *>(lds + kLdsCt);
  for (uint32_t i = tid; i < (kCtBytes + kOtBytes) / 16; i += nt) dst0[i] = src0[i];
  const uint4 *src1 = reinterpret_cast<const uint4 *>(blob + TabCfg<BPW>::ht1);
  uint4 *dst1 = reinterpret_cast<uint4 *>(lds + kLdsHt1);
  for (uint32_t i = tid; i < kHtBytes / 16; i += nt) dst1[i] = src1[i];
  if constexpr (TabCfg<BPW>::ht2_bytes > 0) {
    const uint4 *src2 = reinterpret_cast<const uint4 *>(blob + TabCfg<BPW>::ht2);
    uint4 *dst2 = reinterpret_cast<uint4 *>(lds + kLdsHt2);
    for (uint32_t i = tid; i < TabCfg<BPW>::ht2_bytes / 16; i += nt) dst2[i] = src2[i];
  }
}

// Table walk for one 16-bit index (see glq_tables.h): byte offsets of the
// low and high signed half-vectors within a half table.
__device__ __forceinline__ void walk(uint32_t i, const uint8_t *lds, uint32_t &lo, uint32_t &hi) {
  const uint32_t ip = (i - 1u) & 0xFFFFu;
  const uint32_t e = *reinterpret_cast<const uint16_t *>(lds + kLdsCt + ((ip >> 4) << 1));
  const uint32_t rec = (e >> 5) + ((ip & 15u) >> (e & 31u));
  const uint4 R = *reinterpret_cast<const uint4 *>(lds + kLdsOt + (rec << 4));
  lo = R.y + (__builtin_amdgcn_ubfe(ip, 0, R.x) << 3);
  const uint32_t q = __builtin_popcount(__builtin_amdgcn_ubfe(ip, 0, R.w)) & 1u;
  hi = R.z + ((ip >> R.x) << 3) + (q << 6);
}

__device__ __forceinline__ uint32_t pk_add16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}

// Decode one group into 8 x 16-bit operand values, coordinate t in half t of
// the result (uint4 = 8 halves). 2 bpw: bf16 of v. 3/4 bpw: bf16 of 192 + u
// with u = 4 v (3 bpw) or 8 v (4 bpw).
template <int BPW>
__device__ __forceinline__ uint4 decode_group(uint32_t i1, uint32_t i2, const uint8_t *lds) {
  uint32_t lo, hi;
  walk(i1, lds, lo, hi);
  const uint2 a = *reinterpret_cast<const uint2 *>(lds + kLdsHt1 + lo);
  const uint2 b = *reinterpret_cast<const uint2 *>(lds + kLdsHt1 + hi);
  if constexpr (BPW == 2) {
    (void)i2;
    return make_uint4(a.x, a.y, b.x, b.y);
  } else if constexpr (BPW == 3) {
    const uint4 r = *reinterpret_cast<const uint4 *>(lds + kLdsHt2 + (i2 << 4));
    return make_uint4(pk_add16(a.x, r.x), pk_add16(a.y, r.y), pk_add16(b.x, r.z), pk_add16(b.y, r.w));
  } else {
    uint32_t lo2, hi2;
    walk(i2, lds, lo2, hi2);
    const uint2 c = *reinterpret_cast<const uint2 *>(lds + kLdsHt2 + lo2);
    const uint2 d = *reinterpret_cast<const uint2 *>(lds + kLdsHt2 + hi2);
    return make_uint4(pk_add16(a.x, c.x), pk_add16(a.y, c.y), pk_add16(b.x, d.x), pk_add16(b.y, d.y));
  }
}

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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

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

template <int R>
__device__ __forceinline__ void fwht_pass(float *buf, int b, int lo) {
  const int h = 1 << lo;
  const int nsub = b / R;
  for (int q = threadIdx.x; q < nsub; q += blockDim.x) {
    const int base = (q >> lo) * (h * R) + (q & (h - 1));
    float v[R];
#pragma unroll
    for (int m = 0; m < R; ++m) v[m] = buf[base + m * h];
    fwht_regs<R>(v);
#pragma unroll
    for (int m = 0; m < R; ++m) buf[base + m * h] = v[m];
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
        buf[i] = v;
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
        float v = buf[i] * inv;
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

// row sums of a bf16 [rows][n] array (x already rotated, biased operands need them)
__global__ void __launch_bounds__(256)
row_sums_bf16(const uint16_t *x, int64_t rows, int64_t n, float *rowsum) {
  __shared__ float red[4];
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    float rs = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
      rs += __uint_as_float((uint32_t)x[(size_t)row * n + i] << 16);
    for (int off = 32; off > 0; off >>= 1) rs += __shfl_xor(rs, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = rs;
    __syncthreads();
    if (threadIdx.x == 0) rowsum[row] = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- decode only
template <int BPW, bool OUT_F32>
__global__ void __launch_bounds__(256)
decode_weights_k(const uint16_t *idx1, const void *idx2, const uint8_t *blob, float scale,
                 int64_t groups, void *out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  load_tables<BPW>(lds, blob);
  __syncthreads();
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t i1 = idx1[g];
    const uint32_t i2 = BPW == 2 ? 0u : load_idx2(idx2, g, BPW);
    const uint4 h = decode_group<BPW>(i1, i2, lds);
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    float w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = operand_value<BPW>((hw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
      w[t] = scale * v;                          // one float32 multiply
    }
    if constexpr (OUT_F32) {
      float4 *o = reinterpret_cast<float4 *>(out) + 2 * g;
      o[0] = make_float4(w[0], w[1], w[2], w[3]);
      o[1] = make_float4(w[4], w[5], w[6], w[7]);
    } else {
      uint32_t p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        p[t] = (uint32_t)f32_to_bf16_rne(w[2 * t]) | ((uint32_t)f32_to_bf16_rne(w[2 * t + 1]) << 16);
      reinterpret_cast<uint4 *>(out)[g] = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---------------------------------------------------------------- GEMV (m <= 16)
// Workgroup = 4 waves, one 16-row weight tile n0..n0+15. The k axis is cut in
// chunks of 32 groups (256 inputs); wave w takes chunks w, w+4, ... In a chunk,
// lane l (row j = l & 15, k-slot q = l >> 4) owns groups 32c + 8q .. 32c + 8q + 7
// of weight row n0 + j, and MFMA step s contracts group 32c + 8q + s of every
// slot: A = x~ rows (m = l & 15, zero-padded beyond m), B = decoded weights.
template <int BPW>
__global__ void __launch_bounds__(256)
gemv_bf16(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const uint16_t *xt,
          const float *rowsum, int64_t m, int64_t n, int64_t k, float post, void *out,
          glq_dtype out_dt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + lds_table_bytes<BPW>());
  load_tables<BPW>(lds, blob);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t row = n0 + j;
  const bool row_ok = row < n;
  const int64_t G = k / 8;
  const int64_t chunks = (G + 31) / 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = wave; c < chunks; c += 4) {
    const int64_t g0 = 32 * c + 8 * q;
    uint32_t i1s[8], i2s[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t g = g0 + s;
      const bool ok = row_ok && g < G;
      i1s[s] = ok ? idx1[row * G + g] : 0u;
      i2s[s] = (BPW > 2 && ok) ? load_idx2(idx2, row * G + g, BPW) : 0u;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int64_t g = g0 + s;
      uint4 av = make_uint4(0, 0, 0, 0);
      if (j < m && g < G) av = *reinterpret_cast<const uint4 *>(xt + (size_t)j * k + 8 * g);
      const uint4 bv = decode_group<BPW>(i1s[s], i2s[s], lds);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                    __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }
  }
  // D[r][c]: lane holds rows 4*(lane>>4)+t (activation row), column lane&15 (weight row)
#pragma unroll
  for (int t = 0; t < 4; ++t) red[(wave * 16 + 4 * q + t) * 16 + j] = acc[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 4 * q + t;
      float v = red[(0 * 16 + r) * 16 + j] + red[(1 * 16 + r) * 16 + j] +
                red[(2 * 16 + r) * 16 + j] + red[(3 * 16 + r) * 16 + j];
      if (r < m && row_ok) {
        if (Epi<BPW>::bias != 0.0f) v -= Epi<BPW>::bias * rowsum[r];
        store_out(out, out_dt, (size_t)r * n + row, post * v);
      }
    }
  }
}

// ---------------------------------------------------------------- GEMM (m > 16)
// Tile 128 (m) x 128 (n), 4 waves; wave w owns weight rows n0 + 32w .. +31 for
// all 128 activation rows (8 x 2 MFMA 16x16 tiles). Per k-step of 32 inputs
// the workgroup stages x~[128][32] in LDS; every wave decodes its own 32 x 4
// groups straight into B operands (two per lane).
constexpr int GM_BM = 128, GM_BN = 128, GM_LDA = 40;   // LDA in bf16 (row of 32 + pad 8)

template <int BPW>
__global__ void __launch_bounds__(256)
gemm_bf16(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const uint16_t *xt,
          const float *rowsum, int64_t m, int64_t n, int64_t k, float post, void *out,
          glq_dtype out_dt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t *As = reinterpret_cast<uint16_t *>(lds + lds_table_bytes<BPW>());
  load_tables<BPW>(lds, blob);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * GM_BM;
  const int64_t n0 = (int64_t)blockIdx.x * GM_BN + 32 * wave;
  const int64_t G = k / 8;
  f32x4 acc[8][2];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) acc[a][b2] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t ksteps = (G + 3) / 4;
  for (int64_t ks = 0; ks < ksteps; ++ks) {
    __syncthreads();
    // stage x~[m0 .. m0+127][32 ks .. 32 ks + 31]: 512 16-byte pieces, 2 per thread
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int piece = threadIdx.x + 256 * p;
      const int r = piece >> 2, cq = piece & 3;
      const int64_t gm = m0 + r, g = 4 * ks + cq;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gm < m && g < G) v = *reinterpret_cast<const uint4 *>(xt + (size_t)gm * k + 8 * g);
      *reinterpret_cast<uint4 *>(As + r * GM_LDA + 8 * cq) = v;
    }
    // decode this wave's B operands: columns n0 + 16 t + j, group 4 ks + q
    uint4 bv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t rowi = n0 + 16 * t + j, g = 4 * ks + q;
      const bool ok = rowi < n && g < G;
      const uint32_t i1 = ok ? idx1[rowi * G + g] : 0u;
      const uint32_t i2 = (BPW > 2 && ok) ? load_idx2(idx2, rowi * G + g, BPW) : 0u;
      bv[t] = decode_group<BPW>(i1, i2, lds);
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const uint4 av = *reinterpret_cast<const uint4 *>(As + (16 * a + j) * GM_LDA + 8 * q);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                            __builtin_bit_cast(bf16x8, bv[t]),
                                                            acc[a][t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t col = n0 + 16 * t + j;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = m0 + 16 * a + 4 * q + e;
        if (r < m && col < n) {
          float v = acc[a][t][e];
          if (Epi<BPW>::bias != 0.0f) v -= Epi<BPW>::bias * rowsum[r];
          store_out(out, out_dt, (size_t)r * n + col, post * v);
        }
      }
    }
}

// ---------------------------------------------------------------- float32 path
// One wave per weight row (grid-stride); lanes split the groups of the row;
// up to 4 activation rows per pass (the host loops over passes).
template <int BPW>
__global__ void __launch_bounds__(256)
gemv_f32(const uint16_t *idx1, const void *idx2, const uint8_t *blob, const float *xt,
         int64_t m0, int64_t mc, int64_t n, int64_t k, float scale, void *out, glq_dtype out_dt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  load_tables<BPW>(lds, blob);
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
      if (lane == 0 && r < mc) store_out(out, out_dt, (size_t)(m0 + r) * n + row, scale * t);
    }
  }
}

// ---------------------------------------------------------------- host helpers
thread_local char g_last_error[256] = "";

int hip_status(hipError_t e, const char *where = "launch") {
  if (e == hipSuccess) return GLQ_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return GLQ_ERR_HIP;
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

template <class K>
int allow_lds(K kernel, size_t bytes);

int launch_rht(const void *in, glq_dtype in_dt, void *out, glq_dtype out_dt, int64_t rows,
               int64_t n, const int8_t *signs, int transpose, float *rowsum, hipStream_t st) {
  const int lb = log2_block(n);
  if (lb > kMaxLogBlock) return GLQ_ERR_UNSUPPORTED;
  const int64_t grid = rows < 4096 ? rows : 4096;
  const size_t shm = sizeof(float) << lb;
  const int rc = allow_lds(rht_rows, shm + 1024);
  if (rc) return rc;
  hipLaunchKernelGGL(rht_rows, dim3((unsigned)grid), dim3(256), shm, st, in, in_dt, out, out_dt,
                     rows, n, lb, signs, transpose, rowsum);
  return hip_status(hipGetLastError());
}

// Allow dynamic LDS above the 64 KiB default (gfx950 has 160 KiB per CU).
template <class K>
int allow_lds(K kernel, size_t bytes) {
  if (bytes <= 60 * 1024) return GLQ_OK;
  return hip_status(hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes),
                    "hipFuncSetAttribute");
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
  if ((double)L->n * (double)L->k > 17179869184.0) return GLQ_ERR_UNSUPPORTED;
  return GLQ_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct WsLayout { size_t xt, rowsum, z, total; };

WsLayout ws_layout(int64_t n, int64_t k, int64_t m) {
  WsLayout w;
  w.xt = 0;
  w.rowsum = align256((size_t)m * (size_t)k * 4);
  w.z = w.rowsum + align256((size_t)m * 4);
  w.total = w.z + align256((size_t)m * (size_t)n * 4);
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
                       L->idx1, L->idx2, blob, L->scale, groups, w_out);
  else
    hipLaunchKernelGGL((decode_weights_k<BPW, false>), dim3((unsigned)grid), dim3(256), shm, st,
                       L->idx1, L->idx2, blob, L->scale, groups, w_out);
  return hip_status(hipGetLastError());
}

template <int BPW>
int launch_matmul(const glq_layer *L, const void *xt, glq_dtype x_dt, const float *rowsum, int64_t m,
                  void *out, glq_dtype out_dt, hipStream_t st) {
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
                         blob, reinterpret_cast<const float *>(xt), m0, mc, L->n, L->k, L->scale, out,
                         out_dt);
      int rc = hip_status(hipGetLastError());
      if (rc) return rc;
    }
    return GLQ_OK;
  }
  const float post = L->scale * Epi<BPW>::mul;
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(xt);
  if (m <= 16) {
    const int64_t grid = (L->n + 15) / 16;
    const size_t shm = tab + 4 * 16 * 16 * 4;
    int rc = allow_lds(gemv_bf16<BPW>, shm);
    if (rc) return rc;
    hipLaunchKernelGGL(gemv_bf16<BPW>, dim3((unsigned)grid), dim3(256), shm, st,
                       L->idx1, L->idx2, blob, xb, rowsum, m, L->n, L->k, post, out, out_dt);
  } else {
    const int64_t gx = (L->n + GM_BN - 1) / GM_BN, gy = (m + GM_BM - 1) / GM_BM;
    if (gy > 65535) return GLQ_ERR_UNSUPPORTED;
    const size_t shm = tab + GM_BM * GM_LDA * 2;
    int rc = allow_lds(gemm_bf16<BPW>, shm);
    if (rc) return rc;
    hipLaunchKernelGGL(gemm_bf16<BPW>, dim3((unsigned)gx, (unsigned)gy), dim3(256), shm, st, L->idx1, L->idx2, blob, xb, rowsum, m, L->n, L->k,
                       post, out, out_dt);
  }
  return hip_status(hipGetLastError());
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

  const void *xt_use = x;
  if (x_dt == GLQ_F32) {
    if (in_rht) {
      rc = launch_rht(x, GLQ_F32, xt, GLQ_F32, m, L->k, L->sign_k, 0, nullptr, st);
      if (rc) return rc;
      xt_use = xt;
    }
  } else {
    if (in_rht) {
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
  void *mm_out = out_rht ? (void *)z : y;
  const glq_dtype mm_dt = out_rht ? GLQ_F32 : y_dt;
  switch (L->bpw) {
    case 2: rc = launch_matmul<2>(L, xt_use, x_dt, rowsum, m, mm_out, mm_dt, st); break;
    case 3: rc = launch_matmul<3>(L, xt_use, x_dt, rowsum, m, mm_out, mm_dt, st); break;
    default: rc = launch_matmul<4>(L, xt_use, x_dt, rowsum, m, mm_out, mm_dt, st); break;
  }
  if (rc) return rc;
  if (out_rht) return launch_rht(z, GLQ_F32, y, y_dt, m, L->n, L->sign_n, 1, nullptr, st);
  return GLQ_OK;
}
