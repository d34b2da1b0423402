// glq_encode.cpp -- CPU reference encoder (glq_encode_ref).
//
// "glq 0.1.1" (PyPI), "How it works": weights are rotated by a randomized
// Hadamard transform (item 2) and every group of 8 is mapped to its nearest
// E8 codebook vector (item 1); 3/4 bpw add a residual stage. Decisions the
// page leaves open: s = fp32(sqrt(mean(W~^2))), groups of 8 along k, float64
// squared distances with the lowest index on ties, greedy residual stage with
// C_r = first 2^8 / 2^16 entries scaled by 2^-1 / 2^-2.
//
// Nearest neighbour, exact:
//  1. Closest E8 point (Conway & Sloane, "Sphere Packings, Lattices and
//     Groups", ch. 20: round to D8 and to D8 + 1/2, fix the coordinate-sum
//     parity by re-rounding the worst coordinate, keep the nearer coset).
//     When that point is unique with a margin and lies in the searched part
//     of the codebook it is the answer.
//  2. Otherwise the best point of every sign orbit is found in closed form
//     (signs follow x; half-integer orbits with the wrong parity flip their
//     cheapest coordinate), and every orbit within 1e-9 of the best is
//     searched point by point for the lowest index at the minimum distance.
//
// LDLQ error feedback (glq_encode_ldlq; "How it works", item 3, and GPTQ in
// "Acknowledgments"): the Hessian is rotated like the weights (item 2),
// H~ = V H V^T, damped by damp * mean(diag H~) on the diagonal, and factored
// as H~ = (I + U) D (I + U)^T with U strictly block upper triangular over
// blocks of 8 inputs (from the last block backward: D_j = the diagonal block,
// U_ij = H~_ij D_j^-1, Schur complement of the leading part). Every row is
// then swept block by block along k: T_j = X_j + sum_{i<j} (X_i - X^_i) U_ij
// and X^_j = the same nearest / residual quantiser applied to T_j.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <thread>
#include <unordered_map>
#include <vector>

#include "glq.h"
#include "glq_internal.h"
#include "glq_tables.h"

namespace glq {
namespace {

struct OrbitInfo {
  uint32_t start, count, full;   // full = complete orbit size (2^nnz or 128)
  bool half;
  bool parity_flip;       // half-integer: x8 must be negative when x1..x7 are positive
  double c[8];            // |x|
};

struct Searcher {
  const int8_t *cb = nullptr;            // doubled coordinates
  std::unordered_map<uint64_t, uint32_t> index;
  std::vector<OrbitInfo> orbits;

  static uint64_t key(const int *y) {
    uint64_t k = 0;
    for (int t = 0; t < 8; ++t) k |= (uint64_t)(uint8_t)(int8_t)y[t] << (8 * t);
    return k;
  }

  bool init() {
    cb = codebook_doubled();
    if (!cb) return false;
    index.reserve(kCodebookSize * 2);
    for (uint32_t i = 0; i < kCodebookSize; ++i) {
      int y[8];
      for (int t = 0; t < 8; ++t) y[t] = cb[8 * i + t];
      index.emplace(key(y), i);
    }
    for (uint32_t i = 0; i < kCodebookSize;) {
      OrbitInfo o;
      o.start = i;
      int a[8];
      for (int t = 0; t < 8; ++t) a[t] = std::abs((int)cb[8 * i + t]);
      uint32_t e = i + 1;
      while (e < kCodebookSize) {
        bool same = true;
        for (int t = 0; t < 8; ++t) same &= std::abs((int)cb[8 * e + t]) == a[t];
        if (!same) break;
        ++e;
      }
      o.count = e - i;
      o.half = (a[0] & 1) != 0;
      int s = 0;
      for (int t = 0; t < 8; ++t) { o.c[t] = 0.5 * a[t]; s += a[t]; }
      int nnz = 0;
      for (int t = 0; t < 8; ++t) nnz += a[t] != 0;
      o.full = o.half ? 128u : (1u << nnz);
      o.parity_flip = o.half && (s % 4) != 0;
      orbits.push_back(o);
      i = e;
    }
    return true;
  }

  double dist(const double *x, uint32_t i) const {
    double d = 0.0;
    for (int t = 0; t < 8; ++t) {
      double u = x[t] - 0.5 * cb[8 * i + t];
      d += u * u;
    }
    return d;
  }

  // Nearest D8 point (integer coordinates with even sum); certain = unique with margin.
  static void closest_d8(const double *x, double *f, bool &certain) {
    const double eps = 1e-9;
    double worst = -1.0, second = -1.0;
    int wi = 0;
    double sum = 0.0;
    certain = true;
    for (int t = 0; t < 8; ++t) {
      f[t] = std::nearbyint(x[t]);
      double ad = std::fabs(x[t] - f[t]);
      if (std::fabs(ad - 0.5) <= eps) certain = false;
      if (ad > worst) { second = worst; worst = ad; wi = t; }
      else if (ad > second) second = ad;
      sum += f[t];
    }
    if (std::fmod(std::fabs(sum), 2.0) != 0.0) {
      if (worst - second <= eps) certain = false;
      f[wi] += (x[wi] - f[wi] >= 0.0) ? 1.0 : -1.0;
    }
  }

  // index of the unique nearest lattice point if certain and in [0, limit), else -1
  int64_t lattice_prefilter(const double *x, uint32_t limit) const {
    double a[8], b[8], xs[8];
    bool ca, cbb;
    closest_d8(x, a, ca);
    for (int t = 0; t < 8; ++t) xs[t] = x[t] - 0.5;
    closest_d8(xs, b, cbb);
    double da = 0, db = 0;
    for (int t = 0; t < 8; ++t) {
      b[t] += 0.5;
      da += (x[t] - a[t]) * (x[t] - a[t]);
      db += (x[t] - b[t]) * (x[t] - b[t]);
    }
    if (std::fabs(da - db) <= 1e-9) return -1;
    const double *p = db < da ? b : a;
    if (!(db < da ? cbb : ca)) return -1;
    int y[8];
    for (int t = 0; t < 8; ++t) y[t] = (int)std::lrint(2.0 * p[t]);
    auto it = index.find(key(y));
    if (it == index.end() || it->second >= limit) return -1;
    return (int64_t)it->second;
  }

  // exact minimum squared distance over one whole orbit (closed form)
  static double orbit_min(const OrbitInfo &o, const double *x) {
    double d = 0.0;
    if (!o.half) {
      for (int t = 0; t < 8; ++t) {
        double u = std::fabs(x[t]) - o.c[t];
        d += u * u;
      }
      return d;
    }
    int neg = 0;
    double cheapest = 1e300;
    for (int t = 0; t < 8; ++t) {
      double ax = std::fabs(x[t]);
      double u = ax - o.c[t];
      d += u * u;
      if (x[t] < 0) ++neg;
      cheapest = std::min(cheapest, 4.0 * ax * o.c[t]);
    }
    // with no negatives the point needs x8 < 0 iff parity_flip; each negative
    // toggles that requirement, so the chosen pattern is valid iff neg parity
    // equals parity_flip
    bool valid = (neg & 1) == (o.parity_flip ? 1 : 0);
    return valid ? d : d + cheapest;
  }

  uint32_t nearest(const double *x, uint32_t limit) const {
    int64_t p = lattice_prefilter(x, limit);
    if (p >= 0) return (uint32_t)p;
    double dmin[2048];
    double best = 1e300;
    size_t no = orbits.size();
    for (size_t o = 0; o < no; ++o) {
      const OrbitInfo &ob = orbits[o];
      if (ob.start >= limit) { dmin[o] = 1e300; continue; }
      bool whole = ob.count == ob.full && ob.start + ob.full <= limit;
      double d;
      if (whole) d = orbit_min(ob, x);
      else {
        d = 1e300;
        uint32_t end = std::min<uint32_t>(ob.start + ob.count, limit);
        for (uint32_t i = ob.start; i < end; ++i) d = std::min(d, dist(x, i));
      }
      dmin[o] = d;
      best = std::min(best, d);
    }
    uint32_t arg = 0xFFFFFFFFu;
    double bd = 1e300;
    for (size_t o = 0; o < no; ++o) {
      if (dmin[o] > best + 1e-9) continue;
      const OrbitInfo &ob = orbits[o];
      uint32_t end = std::min<uint32_t>(ob.start + ob.count, limit);
      for (uint32_t i = ob.start; i < end; ++i) {
        double d = dist(x, i);
        if (d < bd || (d == bd && i < arg)) { bd = d; arg = i; }
      }
    }
    return arg;
  }
};

}  // namespace
}  // namespace glq

namespace glq {
namespace {

void fwht(double *v, int64_t b) {
  for (int64_t h = 1; h < b; h <<= 1)
    for (int64_t i = 0; i < b; i += 2 * h)
      for (int64_t j = i; j < i + h; ++j) {
        double a = v[j], c = v[j + h];
        v[j] = a + c;
        v[j + h] = a - c;
      }
}

// V v: sign flips, block Hadamard (b = largest power of two dividing n), / sqrt(b)
void rht_forward(double *v, int64_t n, const int8_t *sigma) {
  int64_t b = n & -n;
  double inv = 1.0 / std::sqrt((double)b);
  for (int64_t i = 0; i < n; ++i) v[i] *= (double)sigma[i];
  for (int64_t o = 0; o < n; o += b) fwht(v + o, b);
  for (int64_t i = 0; i < n; ++i) v[i] *= inv;
}

constexpr int64_t kMaxLdlqK = 16384;

// out = U M V^T in float64 for M [rows][cols] (float or double): every row
// gets V (signs sign_c over cols), then every column gets U (signs sign_r)
template <class T>
void rotate_both(const T *m, int64_t rows, int64_t cols, const int8_t *sign_r, const int8_t *sign_c,
                 int nt, double *out) {
  parallel_for(rows, nt, [&](int64_t r) {
    double *row = out + r * cols;
    for (int64_t c = 0; c < cols; ++c) row[c] = (double)m[r * cols + c];
    rht_forward(row, cols, sign_c);
  });
  const int64_t cblk = 64;
  parallel_for((cols + cblk - 1) / cblk, nt, [&](int64_t cb) {
    std::vector<double> col((size_t)rows);
    int64_t c1 = std::min(cols, (cb + 1) * cblk);
    for (int64_t c = cb * cblk; c < c1; ++c) {
      for (int64_t r = 0; r < rows; ++r) col[r] = out[r * cols + c];
      rht_forward(col.data(), rows, sign_r);
      for (int64_t r = 0; r < rows; ++r) out[r * cols + c] = col[r];
    }
  });
}

}  // namespace
}  // namespace glq

namespace glq {
namespace {

// Block factorisation H = (I + U) D (I + U)^T of a symmetric k x k matrix a
// (row-major, overwritten). Only the block upper part (row block <= column
// block) of a is read and updated. U is returned packed by column block: the
// 8j x 8 block U[0:8j, 8j:8j+8] starts at ublk[32 j (j - 1)]. false when a
// diagonal block of a Schur complement is not positive definite.
bool block_udu(double *a, int64_t k, int nt, std::vector<double> &ublk) {
  const int64_t nb = k / 8;
  ublk.assign((size_t)(32 * nb * (nb - 1)) + 8, 0.0);
  for (int64_t j = nb - 1; j >= 0; --j) {
    const int64_t c0 = 8 * j;
    double d[8][8], l[8][8], inv[8][8];
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) d[r][c] = a[(c0 + std::min(r, c)) * k + c0 + std::max(r, c)];
    // Cholesky d = l l^T (positive definiteness test), then inv = d^-1
    for (int r = 0; r < 8; ++r) {
      for (int c = 0; c <= r; ++c) {
        double v = d[r][c];
        for (int t = 0; t < c; ++t) v -= l[r][t] * l[c][t];
        if (r == c) {
          if (!(v > 0.0) || !std::isfinite(v)) return false;
          l[r][r] = std::sqrt(v);
        } else {
          l[r][c] = v / l[c][c];
        }
      }
      for (int c = r + 1; c < 8; ++c) l[r][c] = 0.0;
    }
    for (int e = 0; e < 8; ++e) {
      double y[8], x[8];
      for (int r = 0; r < 8; ++r) {            // l y = e_e
        double v = r == e ? 1.0 : 0.0;
        for (int t = 0; t < r; ++t) v -= l[r][t] * y[t];
        y[r] = v / l[r][r];
      }
      for (int r = 7; r >= 0; --r) {           // l^T x = y
        double v = y[r];
        for (int t = r + 1; t < 8; ++t) v -= l[t][r] * x[t];
        x[r] = v / l[r][r];
      }
      for (int r = 0; r < 8; ++r) inv[r][e] = x[r];
    }
    if (j == 0) break;
    double *u = ublk.data() + 32 * j * (j - 1);
    // U_i,j = H_i,j D_j^-1 for the rows above block j
    parallel_for(c0, nt > 1 && c0 >= 256 ? nt : 1, [&](int64_t i) {
      const double *hi = a + i * k + c0;
      for (int c = 0; c < 8; ++c) {
        double v = 0.0;
        for (int t = 0; t < 8; ++t) v += hi[t] * inv[t][c];
        u[i * 8 + c] = v;
      }
    });
    // Schur complement: a[i][l] -= U_i,j . H_l,j over the block upper part
    parallel_for(j, nt > 1 && j >= 8 ? nt : 1, [&](int64_t ib) {
      for (int64_t i = 8 * ib; i < 8 * ib + 8; ++i) {
        const double *ui = u + i * 8;
        double *ai = a + i * k;
        for (int64_t l2 = 8 * ib; l2 < c0; ++l2) {
          const double *hl = a + l2 * k + c0;
          double v = 0.0;
          for (int c = 0; c < 8; ++c) v += ui[c] * hl[c];
          ai[l2] -= v;
        }
      }
    });
  }
  return true;
}

int encode_impl(const float *w, int64_t n, int64_t k, int32_t bpw,
                const int8_t *sign_n, const int8_t *sign_k,
                float scale_in, float *scale_out,
                uint16_t *idx1_out, void *idx2_out, int32_t nthreads,
                float *row_scale_out, const double *hessian, double damp) {
  if (!w || !sign_n || !sign_k || !idx1_out) return GLQ_ERR_ARG;
  if (n < 1 || k < 8 || k % 8 != 0) return GLQ_ERR_ARG;
  if (bpw != 2 && bpw != 3 && bpw != 4) return GLQ_ERR_ARG;
  if (bpw > 2 && !idx2_out) return GLQ_ERR_ARG;
  if (!(scale_in <= 0.0f || std::isfinite(scale_in))) return GLQ_ERR_ARG;
  if ((double)n * (double)k > 4.0e9) return GLQ_ERR_UNSUPPORTED;
  if (hessian && (!std::isfinite(damp) || damp < 0.0)) return GLQ_ERR_ARG;
  if (hessian && k > kMaxLdlqK) return GLQ_ERR_UNSUPPORTED;
  for (int64_t i = 0; i < n; ++i) if (sign_n[i] != 1 && sign_n[i] != -1) return GLQ_ERR_ARG;
  for (int64_t i = 0; i < k; ++i) if (sign_k[i] != 1 && sign_k[i] != -1) return GLQ_ERR_ARG;
  const int64_t nk = n * k;
  for (int64_t i = 0; i < nk; ++i) if (!std::isfinite(w[i])) return GLQ_ERR_ARG;
  if (hessian)
    for (int64_t i = 0; i < k * k; ++i) if (!std::isfinite(hessian[i])) return GLQ_ERR_ARG;

  static Searcher S;
  static std::once_flag once;
  static bool ok = false;
  std::call_once(once, [] { ok = S.init(); });
  if (!ok) return GLQ_ERR_UNSUPPORTED;

  int nt = nthreads > 0 ? nthreads : (int)std::max(1u, std::thread::hardware_concurrency());

  // rotated, damped Hessian and its block factorisation (before any output)
  std::vector<double> ublk;
  if (hessian) {
    std::vector<double> ht((size_t)(k * k));
    rotate_both(hessian, k, k, sign_k, sign_k, nt, ht.data());
    long double dsum = 0.0L;
    for (int64_t i = 0; i < k; ++i) dsum += ht[i * k + i];
    const double add = damp * (double)(dsum / (long double)k);
    for (int64_t i = 0; i < k; ++i) ht[i * k + i] += add;
    if (!block_udu(ht.data(), k, nt, ublk)) return GLQ_ERR_ARG;
  }

  // W~ = U W V^T in float64
  std::vector<double> wt((size_t)nk);
  rotate_both(w, n, k, sign_n, sign_k, nt, wt.data());

  // scales: one global s, or one per row (row r divided by srow[r])
  std::vector<float> srow((size_t)n, 1.0f);
  float s = 1.0f;
  const bool per_row = row_scale_out != nullptr;
  if (per_row || scale_in <= 0.0f) {
    // mean of squares with per-row long double partial sums
    std::vector<long double> part((size_t)n);
    parallel_for(n, nt, [&](int64_t r) {
      long double acc = 0.0L;
      const double *row = wt.data() + r * k;
      for (int64_t c = 0; c < k; ++c) acc += (long double)row[c] * row[c];
      part[r] = acc;
    });
    if (per_row) {
      for (int64_t r = 0; r < n; ++r) {
        const double ms = (double)(part[r] / (long double)k);
        srow[r] = ms == 0.0 ? 1.0f : (float)std::sqrt(ms);
        row_scale_out[r] = srow[r];
      }
    } else {
      long double tot = 0.0L;
      for (int64_t r = 0; r < n; ++r) tot += part[r];
      const double ms = (double)(tot / (long double)nk);
      s = ms == 0.0 ? 1.0f : (float)std::sqrt(ms);
    }
  } else {
    s = scale_in;
  }
  if (scale_out) *scale_out = s;
  if (!per_row)
    for (int64_t r = 0; r < n; ++r) srow[r] = s;

  const int64_t g = k / 8;
  const uint32_t rlimit = bpw == 3 ? 256u : kCodebookSize;
  const double rmul = bpw == 3 ? 2.0 : 4.0;
  const int8_t *cb = S.cb;
  // Q of one target vector: writes the indices and the exact decoded vector
  auto quantise = [&](const double *x, int64_t r, int64_t q, double *v) {
    uint32_t i1 = S.nearest(x, kCodebookSize);
    idx1_out[r * g + q] = (uint16_t)i1;
    for (int t = 0; t < 8; ++t) v[t] = 0.5 * cb[8 * i1 + t];
    if (bpw > 2) {
      double rr[8];
      for (int t = 0; t < 8; ++t) rr[t] = (x[t] - v[t]) * rmul;
      uint32_t i2 = S.nearest(rr, rlimit);
      if (bpw == 3) ((uint8_t *)idx2_out)[r * g + q] = (uint8_t)i2;
      else ((uint16_t *)idx2_out)[r * g + q] = (uint16_t)i2;
      for (int t = 0; t < 8; ++t) v[t] += 0.5 * cb[8 * i2 + t] / rmul;
    }
  };
  if (!hessian) {
    parallel_for(n, nt, [&](int64_t r) {
      for (int64_t q = 0; q < g; ++q) {
        double x[8], v[8];
        for (int t = 0; t < 8; ++t) x[t] = wt[r * k + 8 * q + t] / (double)srow[r];
        quantise(x, r, q, v);
      }
    });
    return GLQ_OK;
  }
  // LDLQ sweep, rows in tiles of kTile so every U block read serves kTile rows
  constexpr int64_t kTile = 16;
  parallel_for((n + kTile - 1) / kTile, nt, [&](int64_t tile) {
    const int64_t r0 = tile * kTile, nr = std::min(kTile, n - r0);
    std::vector<double> x((size_t)(kTile * k)), e((size_t)(kTile * k));
    for (int64_t a = 0; a < nr; ++a)
      for (int64_t c = 0; c < k; ++c) x[a * k + c] = wt[(r0 + a) * k + c] / (double)srow[r0 + a];
    for (int64_t q = 0; q < g; ++q) {
      double t[kTile][8];
      for (int64_t a = 0; a < nr; ++a)
        for (int c = 0; c < 8; ++c) t[a][c] = 0.0;
      const double *u = ublk.data() + 32 * q * (q - 1);
      for (int64_t i = 0; i < 8 * q; ++i) {
        const double *ui = u + i * 8;
        for (int64_t a = 0; a < nr; ++a) {
          const double ei = e[a * k + i];
          for (int c = 0; c < 8; ++c) t[a][c] += ei * ui[c];
        }
      }
      for (int64_t a = 0; a < nr; ++a) {
        double tv[8], v[8];
        for (int c = 0; c < 8; ++c) tv[c] = x[a * k + 8 * q + c] + t[a][c];
        quantise(tv, r0 + a, q, v);
        for (int c = 0; c < 8; ++c) e[a * k + 8 * q + c] = x[a * k + 8 * q + c] - v[c];
      }
    }
  });
  return GLQ_OK;
}

}  // namespace

void rotate_weights_f64(const float *w, int64_t n, int64_t k, const int8_t *sign_n,
                        const int8_t *sign_k, int nthreads, double *out) {
  rotate_both(w, n, k, sign_n, sign_k, nthreads, out);
}

}  // namespace glq

extern "C" int glq_encode_ref(const float *w, int64_t n, int64_t k, int32_t bpw,
                              const int8_t *sign_n, const int8_t *sign_k,
                              float scale_in, float *scale_out,
                              uint16_t *idx1_out, void *idx2_out, int32_t nthreads,
                              float *row_scale_out) {
  return glq::encode_impl(w, n, k, bpw, sign_n, sign_k, scale_in, scale_out, idx1_out, idx2_out,
                          nthreads, row_scale_out, nullptr, 0.0);
}

extern "C" int glq_encode_ldlq(const float *w, int64_t n, int64_t k, int32_t bpw,
                               const int8_t *sign_n, const int8_t *sign_k,
                               const double *hessian, double damp,
                               float scale_in, float *scale_out,
                               uint16_t *idx1_out, void *idx2_out, int32_t nthreads,
                               float *row_scale_out) {
  if (!hessian) return GLQ_ERR_ARG;
  return glq::encode_impl(w, n, k, bpw, sign_n, sign_k, scale_in, scale_out, idx1_out, idx2_out,
                          nthreads, row_scale_out, hessian, damp);
}
