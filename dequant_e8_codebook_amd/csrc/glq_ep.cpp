// glq_ep.cpp -- CPU side of the entropy-coded E8 lattice format: encoder
// (glq_ep_encode) and decode-table builder (glq_ep_build_lut).
//
// "Transformers Proposes EntroPack Integration ..." (first two paragraphs):
// per-row normalised E8 lattice quantisation, a conditional probability model
// and entropy coding, in independently decodable blocks. The page states no
// formulas; the format is defined in glq.h:
//  - s_r = fp32(sqrt(mean_j W~[r,j]^2)); z = 2 * nearest E8 point to
//    (W~[r] / s_r) / step over the whole lattice (Conway & Sloane,
//    "Sphere Packings, Lattices and Groups", ch. 20: nearest D8 point of x and
//    of x - 1/2, keep the nearer coset).
//  - 8 symbols per group under 5 tables: z_1; (z_c - b)/2 given the coset b;
//    (z_8 - t)/4 with t the residue the even-sum rule leaves.
//  - static frequencies per table, 11-bit precision: each seen symbol gets
//    1 + floor(c (2048 - nz) / N); the rest go one each to the largest
//    remainders, ties to the smaller value.
//  - range ANS (J. Duda, "Asymmetric numeral systems", 2013): 32-bit state
//    in [2^16, 2^32), 16-bit words; a block's 64 lanes are coded so that a
//    decoder stepping them in lockstep reads the words of one step in lane
//    order (encode in reverse: steps backward, lanes high to low, then
//    reverse the emitted words).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "glq.h"
#include "glq_internal.h"

namespace glq {
namespace {

constexpr int kLanes = GLQ_EP_LANES;
constexpr int kTables = GLQ_EP_TABLES;
constexpr int kMaxSyms = GLQ_EP_MAX_SYMS;
constexpr uint32_t kPrecBits = 11;
constexpr uint32_t kM = 1u << kPrecBits;
constexpr uint32_t kL = 1u << 16;

// nearest D8 point (integers, even sum): round half to even, then move the
// first coordinate with the largest rounding error if the sum is odd
void closest_d8(const double *x, double *f) {
  double worst = -1.0;
  int wi = 0;
  double sum = 0.0;
  for (int t = 0; t < 8; ++t) {
    f[t] = std::nearbyint(x[t]);
    const double ad = std::fabs(x[t] - f[t]);
    if (ad > worst) { worst = ad; wi = t; }
    sum += f[t];
  }
  if (std::fmod(std::fabs(sum), 2.0) != 0.0) f[wi] += (x[wi] - f[wi] >= 0.0) ? 1.0 : -1.0;
}

// doubled nearest E8 point; the integer coset on equal distances
void closest_e8_doubled(const double *x, int64_t *z) {
  double a[8], b[8], xs[8];
  closest_d8(x, a);
  for (int t = 0; t < 8; ++t) xs[t] = x[t] - 0.5;
  closest_d8(xs, b);
  double da = 0.0, db = 0.0;
  for (int t = 0; t < 8; ++t) {
    b[t] += 0.5;
    da += (x[t] - a[t]) * (x[t] - a[t]);
    db += (x[t] - b[t]) * (x[t] - b[t]);
  }
  const double *p = db < da ? b : a;
  for (int t = 0; t < 8; ++t) z[t] = (int64_t)std::llrint(2.0 * p[t]);
}

int64_t floor_div(int64_t a, int64_t d) {   // d > 0
  int64_t q = a / d;
  return (a % d != 0 && a < 0) ? q - 1 : q;
}

// the 8 (table, value) pairs of one group
void group_symbols(const int64_t *z, int *tab, int64_t *val) {
  const int64_t b = z[0] & 1;
  tab[0] = 0;
  val[0] = z[0];
  int64_t s7 = z[0];
  for (int c = 1; c < 7; ++c) {
    tab[c] = 1 + (int)b;
    val[c] = floor_div(z[c] - b, 2);
    s7 += z[c];
  }
  const int64_t t = ((-s7) % 4 + 4) % 4;
  tab[7] = 3 + (int)b;
  val[7] = floor_div(z[7] - t, 4);
}

void normalise(const std::vector<int64_t> &c, uint16_t *f) {
  const size_t ns = c.size();
  int64_t nz = 0, tot = 0;
  for (size_t s = 0; s < ns; ++s) { nz += c[s] > 0; tot += c[s]; }
  std::vector<int64_t> frac(ns, 0);
  int64_t sum = 0;
  for (size_t s = 0; s < ns; ++s) {
    f[s] = 0;
    if (c[s] > 0) {
      const int64_t num = c[s] * ((int64_t)kM - nz);
      f[s] = (uint16_t)(1 + num / tot);
      frac[s] = num % tot;
      sum += f[s];
    }
  }
  std::vector<size_t> order;
  for (size_t s = 0; s < ns; ++s) if (c[s] > 0) order.push_back(s);
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return frac[a] > frac[b]; });
  for (int64_t r = 0, rem = (int64_t)kM - sum; r < rem; ++r) f[order[(size_t)r]] += 1;
}

}  // namespace
}  // namespace glq

extern "C" int glq_ep_encode(const float *w, int64_t n, int64_t k, const int8_t *sign_n,
                             const int8_t *sign_k, float step, int32_t lane_groups, int32_t nthreads,
                             float *row_scale_out, glq_ep_model *model_out, uint32_t *states_out,
                             uint32_t *offsets_out, uint16_t *words_out, int64_t words_capacity,
                             int64_t *words_written) {
  using namespace glq;
  if (!w || !sign_n || !sign_k || !row_scale_out || !model_out || !states_out || !offsets_out ||
      !words_written)
    return GLQ_ERR_ARG;
  if (n < 1 || k < 8 || k % 8 != 0 || lane_groups < 1) return GLQ_ERR_ARG;
  if (!(step > 0.0f) || !std::isfinite(step)) return GLQ_ERR_ARG;
  if (words_capacity < 0 || (words_capacity > 0 && !words_out)) return GLQ_ERR_ARG;
  const int64_t g = k / 8, total = n * g;
  if ((double)n * (double)k / 8.0 >= 2147483648.0) return GLQ_ERR_UNSUPPORTED;
  for (int64_t i = 0; i < n; ++i) if (sign_n[i] != 1 && sign_n[i] != -1) return GLQ_ERR_ARG;
  for (int64_t i = 0; i < k; ++i) if (sign_k[i] != 1 && sign_k[i] != -1) return GLQ_ERR_ARG;
  for (int64_t i = 0; i < n * k; ++i) if (!std::isfinite(w[i])) return GLQ_ERR_ARG;
  const int nt = nthreads > 0 ? nthreads : (int)std::max(1u, std::thread::hardware_concurrency());

  std::vector<double> wt((size_t)(n * k));
  rotate_weights_f64(w, n, k, sign_n, sign_k, nt, wt.data());

  // per-row scales, then the doubled lattice points and their symbols
  std::vector<float> srow((size_t)n);
  parallel_for(n, nt, [&](int64_t r) {
    long double acc = 0.0L;
    const double *row = wt.data() + r * k;
    for (int64_t c = 0; c < k; ++c) acc += (long double)row[c] * row[c];
    const double ms = (double)(acc / (long double)k);
    srow[(size_t)r] = ms == 0.0 ? 1.0f : (float)std::sqrt(ms);
  });
  std::vector<int64_t> vals((size_t)(total * 8));
  std::vector<uint8_t> tabs((size_t)(total * 8));
  const double dstep = (double)step;
  parallel_for(n, nt, [&](int64_t r) {
    for (int64_t q = 0; q < g; ++q) {
      double x[8];
      int64_t z[8];
      int tb[8];
      for (int t = 0; t < 8; ++t) x[t] = (wt[(size_t)(r * k + 8 * q + t)] / (double)srow[(size_t)r]) / dstep;
      closest_e8_doubled(x, z);
      const size_t o = (size_t)((r * g + q) * 8);
      group_symbols(z, tb, &vals[o]);
      for (int t = 0; t < 8; ++t) tabs[o + t] = (uint8_t)tb[t];
    }
  });

  // model: value span and frequencies of every table
  int64_t lo[kTables], hi[kTables];
  for (int t = 0; t < kTables; ++t) { lo[t] = INT64_MAX; hi[t] = INT64_MIN; }
  for (size_t i = 0; i < vals.size(); ++i) {
    lo[tabs[i]] = std::min(lo[tabs[i]], vals[i]);
    hi[tabs[i]] = std::max(hi[tabs[i]], vals[i]);
  }
  std::memset(model_out, 0, sizeof(*model_out));
  for (int t = 0; t < kTables; ++t) {
    if (lo[t] > hi[t]) continue;
    if (hi[t] - lo[t] + 1 > kMaxSyms) return GLQ_ERR_UNSUPPORTED;
    if (lo[t] < INT32_MIN || hi[t] > INT32_MAX) return GLQ_ERR_UNSUPPORTED;
    model_out->vmin[t] = (int32_t)lo[t];
    model_out->nsym[t] = (int32_t)(hi[t] - lo[t] + 1);
  }
  {
    std::vector<int64_t> cnt[kTables];
    for (int t = 0; t < kTables; ++t) cnt[t].assign((size_t)model_out->nsym[t], 0);
    for (size_t i = 0; i < vals.size(); ++i) cnt[tabs[i]][(size_t)(vals[i] - lo[tabs[i]])] += 1;
    for (int t = 0; t < kTables; ++t)
      if (model_out->nsym[t]) normalise(cnt[t], model_out->freq[t]);
  }
  uint32_t cum[kTables][kMaxSyms];
  for (int t = 0; t < kTables; ++t) {
    uint32_t a = 0;
    for (int s = 0; s < kMaxSyms; ++s) { cum[t][s] = a; a += model_out->freq[t][s]; }
  }
  for (int64_t r = 0; r < n; ++r) row_scale_out[r] = srow[(size_t)r];

  // blocks, coded independently
  const int64_t bg = (int64_t)kLanes * lane_groups;
  const int64_t nb = (total + bg - 1) / bg;
  std::vector<std::vector<uint16_t>> out((size_t)nb);
  parallel_for(nb, nt, [&](int64_t blk) {
    const int64_t g0 = blk * bg, ng = std::min(bg, total - g0);
    const int64_t pmax = (ng + kLanes - 1) / kLanes;
    uint32_t x[kLanes];
    for (int l = 0; l < kLanes; ++l) x[l] = kL;
    std::vector<uint16_t> &o = out[(size_t)blk];
    o.reserve((size_t)(ng * 4));
    for (int64_t p = pmax - 1; p >= 0; --p)
      for (int c = 7; c >= 0; --c)
        for (int l = kLanes - 1; l >= 0; --l) {
          const int64_t j = p * kLanes + l;
          if (j >= ng) continue;
          const size_t i = (size_t)((g0 + j) * 8 + c);
          const int t = tabs[i];
          const int s = (int)(vals[i] - lo[t]);
          const uint32_t f = model_out->freq[t][s];
          uint32_t xs = x[l];
          if ((uint64_t)xs >= ((uint64_t)f << (32 - kPrecBits))) {   // at most one word: then xs < 2^16
            o.push_back((uint16_t)(xs & 0xFFFFu));
            xs >>= 16;
          }
          x[l] = ((xs / f) << kPrecBits) + (xs % f) + cum[t][s];
        }
    std::reverse(o.begin(), o.end());
    for (int l = 0; l < kLanes; ++l) states_out[blk * kLanes + l] = x[l];
  });
  int64_t nw = 0;
  for (int64_t b = 0; b < nb; ++b) {
    offsets_out[b] = (uint32_t)nw;
    nw += (int64_t)out[(size_t)b].size();
    if (nw > 0xFFFFFFFFll) return GLQ_ERR_UNSUPPORTED;
  }
  offsets_out[nb] = (uint32_t)nw;
  *words_written = nw;
  if (nw > words_capacity) return GLQ_ERR_WORKSPACE;
  for (int64_t b = 0; b < nb; ++b)
    if (!out[(size_t)b].empty())
      std::memcpy(words_out + offsets_out[b], out[(size_t)b].data(), out[(size_t)b].size() * 2);
  return GLQ_OK;
}

extern "C" int glq_ep_build_lut(const glq_ep_model *model, void *lut_out, size_t lut_bytes) {
  using namespace glq;
  if (!model || !lut_out || lut_bytes < (size_t)GLQ_EP_LUT_BYTES) return GLQ_ERR_ARG;
  for (int t = 0; t < kTables; ++t) {
    if (model->nsym[t] < 0 || model->nsym[t] > kMaxSyms) return GLQ_ERR_ARG;
    if (model->nsym[t] == 0) continue;
    uint32_t sum = 0;
    for (int s = 0; s < model->nsym[t]; ++s) sum += model->freq[t][s];
    if (sum != kM) return GLQ_ERR_ARG;
  }
  uint8_t *out = (uint8_t *)lut_out;
  std::memset(out, 0, (size_t)GLQ_EP_LUT_BYTES);
  std::memcpy(out, model->vmin, sizeof(model->vmin));
  uint32_t *lut = (uint32_t *)(out + 64);
  for (int t = 0; t < kTables; ++t) {
    uint32_t c = 0;
    for (int s = 0; s < model->nsym[t]; ++s) {
      const uint32_t f = model->freq[t][s];
      for (uint32_t u = 0; u < f; ++u)
        lut[t * kM + c + u] = (uint32_t)s | (f << 8) | (u << 20);
      c += f;
    }
  }
  return GLQ_OK;
}
