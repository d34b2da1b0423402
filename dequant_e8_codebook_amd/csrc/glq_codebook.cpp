// glq_codebook.cpp -- the E8 codebook in the stated order and its decode tables.
//
// "glq 0.1.1" (PyPI), "How it works", item 1: the codebook holds 65,536
// vectors from the first 7 shells of E8. Format choices the page leaves open:
// standard coordinates (all integer or all half-integer, even sum), the origin
// counted as shell 0, and the order ascending on
//   (|x|^2, -orbit size, max|x_i|, |x| lexicographic, sign counter j)
// with orbit = points sharing |x| (2^nnz points when integer, 128 when
// half-integer), j over the nonzero coordinates in order (integer points) or
// over x1..x7 (half-integer points, the sign of x8 fixed by parity).
//
// Points are held doubled, y = 2x in int8.
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "glq.h"
#include "glq_internal.h"
#include "glq_tables.h"

namespace glq {
namespace {

struct Point {
  std::array<int8_t, 8> y;
  int norm4;      // sum y^2 = 4 |x|^2
  int size;       // orbit size
  int maxabs;
  uint32_t j;     // sign counter
};

bool in_e8_doubled(const int8_t *y) {
  bool all_even = true, all_odd = true;
  int sum = 0;
  for (int t = 0; t < 8; ++t) {
    int v = y[t];
    if (v & 1) all_even = false; else all_odd = false;
    sum += v;
  }
  return (all_even || all_odd) && ((sum % 4) + 4) % 4 == 0;
}

Point make_point(const int8_t *y) {
  Point p;
  int nnz = 0;
  p.norm4 = 0;
  p.maxabs = 0;
  for (int t = 0; t < 8; ++t) {
    p.y[t] = y[t];
    int a = y[t] < 0 ? -y[t] : y[t];
    p.norm4 += a * a;
    p.maxabs = std::max(p.maxabs, a);
    nnz += a != 0;
  }
  bool half = (y[0] & 1) != 0;
  p.size = half ? 128 : (1 << nnz);
  p.j = 0;
  if (half) {
    for (int t = 0; t < 7; ++t) if (y[t] < 0) p.j |= 1u << t;
  } else {
    int r = 0;
    for (int t = 0; t < 8; ++t) {
      if (y[t] != 0) {
        if (y[t] < 0) p.j |= 1u << r;
        ++r;
      }
    }
  }
  return p;
}

bool key_less(const Point &a, const Point &b) {
  if (a.norm4 != b.norm4) return a.norm4 < b.norm4;
  if (a.size != b.size) return a.size > b.size;            // larger orbits first
  if (a.maxabs != b.maxabs) return a.maxabs < b.maxabs;
  for (int t = 0; t < 8; ++t) {
    int x = std::abs(a.y[t]), z = std::abs(b.y[t]);
    if (x != z) return x < z;
  }
  return a.j < b.j;
}

std::vector<Point> build_points() {
  std::vector<Point> pts;
  pts.reserve(120000);
  int8_t y[8];
  // even doubled coordinates in [-6, 6], odd in [-5, 5]: |x_i| <= 3 covers |x|^2 <= 12
  for (int parity = 0; parity < 2; ++parity) {
    const int lo = parity ? -5 : -6, hi = parity ? 5 : 6;
    int idx[8];
    for (int t = 0; t < 8; ++t) idx[t] = lo;
    while (true) {
      for (int t = 0; t < 8; ++t) y[t] = (int8_t)idx[t];
      int n4 = 0;
      for (int t = 0; t < 8; ++t) n4 += idx[t] * idx[t];
      if (n4 <= 48 && in_e8_doubled(y)) pts.push_back(make_point(y));
      int t = 7;
      while (t >= 0) {
        idx[t] += 2;
        if (idx[t] <= hi) break;
        idx[t] = lo;
        --t;
      }
      if (t < 0) break;
    }
  }
  std::sort(pts.begin(), pts.end(), key_less);
  pts.resize(kCodebookSize);
  return pts;
}

struct Orbit {
  uint32_t start;   // first index i
  uint32_t count;   // entries inside the codebook
  uint32_t size;    // full orbit size
  bool half;
  std::array<int, 8> a;   // |y|
};

uint64_t abs_key4(const int *a) {
  return (uint64_t)a[0] | ((uint64_t)a[1] << 8) | ((uint64_t)a[2] << 16) | ((uint64_t)a[3] << 24);
}

uint16_t bf16_of_half(int y) {  // bf16 bits of y / 2 (exact: |y| <= 6)
  float f = 0.5f * (float)y;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

struct Tables {
  std::vector<Point> pts;
  std::vector<Orbit> orbits;
  std::vector<uint8_t> blob;      // GLQ_CB_DEVICE
  std::vector<int8_t> flat;       // GLQ_CB_INT8_2X
  bool ok = false;
};

// Signed half-vectors: y values of 4 coordinates.
struct HalfTable {
  std::vector<std::array<int, 4>> entries;
  std::map<uint64_t, uint32_t> natural;   // abs pattern -> first entry
  std::map<uint64_t, uint32_t> qblock;    // half-integer abs pattern -> first entry (24 entries)

  uint32_t natural_block(const int *a) {
    uint64_t key = abs_key4(a);
    auto it = natural.find(key);
    if (it != natural.end()) return it->second;
    int pos[4], nnz = 0;
    for (int t = 0; t < 4; ++t) if (a[t]) pos[nnz++] = t;
    uint32_t base = (uint32_t)entries.size();
    for (uint32_t s = 0; s < (1u << nnz); ++s) {
      std::array<int, 4> e{a[0], a[1], a[2], a[3]};
      for (int r = 0; r < nnz; ++r) if (s >> r & 1) e[pos[r]] = -e[pos[r]];
      entries.push_back(e);
    }
    natural[key] = base;
    return base;
  }

  // Entry e in [0, 24): q = (e >> 3) & 1, j3 = e & 7 gives the signs of
  // coordinates 0..2; coordinate 3 is negative iff q xor parity(j3) (the
  // parity constant P = 0; P = 1 orbits start 8 entries later).
  uint32_t q_block(const int *a) {
    uint64_t key = abs_key4(a);
    auto it = qblock.find(key);
    if (it != qblock.end()) return it->second;
    uint32_t base = (uint32_t)entries.size();
    for (uint32_t e = 0; e < 24; ++e) {
      uint32_t q = (e >> 3) & 1, j3 = e & 7;
      std::array<int, 4> v{a[0], a[1], a[2], a[3]};
      for (int t = 0; t < 3; ++t) if (j3 >> t & 1) v[t] = -v[t];
      uint32_t par = (j3 ^ (j3 >> 1) ^ (j3 >> 2)) & 1;
      if (q ^ par) v[3] = -v[3];
      entries.push_back(v);
    }
    qblock[key] = base;
    return base;
  }
};

void put16(uint8_t *p, uint16_t v) { std::memcpy(p, &v, 2); }
void put32(uint8_t *p, uint32_t v) { std::memcpy(p, &v, 4); }

bool build_tables(Tables &T) {
  T.pts = build_points();
  const auto &P = T.pts;

  // flat form
  T.flat.resize(kCodebookSize * 8);
  for (uint32_t i = 0; i < kCodebookSize; ++i)
    for (int t = 0; t < 8; ++t) T.flat[i * 8 + t] = P[i].y[t];

  // orbits (runs of equal |y|), the origin included as orbit 0
  for (uint32_t i = 0; i < kCodebookSize;) {
    Orbit o;
    o.start = i;
    for (int t = 0; t < 8; ++t) o.a[t] = std::abs(P[i].y[t]);
    o.half = (P[i].y[0] & 1) != 0;
    o.size = (uint32_t)P[i].size;
    uint32_t e = i;
    while (e < kCodebookSize) {
      bool same = true;
      for (int t = 0; t < 8; ++t) same &= std::abs(P[e].y[t]) == o.a[t];
      if (!same) break;
      ++e;
    }
    o.count = e - i;
    T.orbits.push_back(o);
    i = e;
  }

  HalfTable H;
  // records: one per orbit except the origin, in order; then 16 for the last chunk
  struct Rec { uint32_t r_lo, lo_off, hi_off, qw; };
  std::vector<Rec> recs;
  std::vector<uint32_t> rec_of_orbit(T.orbits.size(), 0xFFFFFFFFu);
  auto make_rec = [&](const Orbit &o) {
    Rec r;
    int lo[4] = {o.a[0], o.a[1], o.a[2], o.a[3]};
    int hi[4] = {o.a[4], o.a[5], o.a[6], o.a[7]};
    uint32_t sp = (o.start - 1u) & 0xFFFFu;       // start in i'
    if (o.half) {
      uint32_t par = 0;
      for (int t = 0; t < 8; ++t) par += (uint32_t)o.a[t];
      uint32_t P8 = (par % 4) != 0;               // x8 negative when x1..x7 positive
      r.r_lo = 4;
      r.lo_off = 8u * H.natural_block(lo);
      uint32_t hb = 8u * H.q_block(hi) + 64u * P8;
      r.hi_off = hb - 8u * (sp >> 4);
      r.qw = 4;
    } else {
      int nlo = 0;
      for (int t = 0; t < 4; ++t) nlo += lo[t] != 0;
      r.r_lo = (uint32_t)nlo;
      r.lo_off = 8u * H.natural_block(lo);
      uint32_t hb = 8u * H.natural_block(hi);
      r.hi_off = hb - 8u * (sp >> r.r_lo);
      r.qw = 0;
    }
    return r;
  };
  for (size_t oi = 1; oi < T.orbits.size(); ++oi) {
    rec_of_orbit[oi] = (uint32_t)recs.size();
    recs.push_back(make_rec(T.orbits[oi]));
  }
  Rec origin_rec;
  {
    Orbit o = T.orbits[0];          // the origin: start 0 -> i' = 65535
    int z[4] = {0, 0, 0, 0};
    origin_rec.r_lo = 0;
    origin_rec.lo_off = 8u * H.natural_block(z);
    origin_rec.hi_off = 8u * H.natural_block(z) - 8u * ((o.start - 1u) & 0xFFFFu);
    origin_rec.qw = 0;
  }

  // orbit containing each index
  std::vector<uint32_t> orbit_of(kCodebookSize);
  for (size_t oi = 0; oi < T.orbits.size(); ++oi)
    for (uint32_t i = T.orbits[oi].start; i < T.orbits[oi].start + T.orbits[oi].count; ++i)
      orbit_of[i] = (uint32_t)oi;

  std::vector<uint16_t> ct(kChunks);
  for (uint32_t c = 0; c < kChunks; ++c) {
    uint32_t i0 = 16 * c + 1;                      // i of slot 0 (i' = 16c)
    if (c == kChunks - 1) {
      uint32_t first = (uint32_t)recs.size();
      for (uint32_t s = 0; s < 16; ++s) {
        uint32_t ip = 16 * c + s;
        Rec r = ip == 0xFFFFu ? origin_rec : recs[rec_of_orbit[orbit_of[ip + 1]]];
        recs.push_back(r);
      }
      ct[c] = (uint16_t)((first << 5) | 0u);
      continue;
    }
    const Orbit &o = T.orbits[orbit_of[i0]];
    uint32_t ls = 4;
    if (o.size < 16) {
      ls = 0;
      while ((1u << ls) < o.size) ++ls;
    }
    ct[c] = (uint16_t)((rec_of_orbit[orbit_of[i0]] << 5) | ls);
  }
  if (recs.size() > kMaxRecords || H.entries.size() > kMaxHalves) return false;

  // blob
  T.blob.assign(kBlobBytes, 0);
  uint8_t *b = T.blob.data();
  put32(b + 0, kMagic0);
  put32(b + 4, kFormatVersion);
  put32(b + 8, (uint32_t)recs.size());
  put32(b + 12, (uint32_t)H.entries.size());
  for (uint32_t c = 0; c < kChunks; ++c) put16(b + kCtOff + 2 * c, ct[c]);
  for (size_t r = 0; r < recs.size(); ++r) {
    const int32_t hs = (int32_t)recs[r].hi_off;       // may be negative (wraps in uint32)
    if (recs[r].r_lo > 31 || recs[r].qw > 31 || recs[r].lo_off >= (1u << 24) || hs < -(1 << 23) || hs >= (1 << 23))
      return false;
    uint8_t *p = b + kOtOff + 8 * r;
    put32(p + 0, recs[r].r_lo | (recs[r].lo_off << 8));
    put32(p + 4, recs[r].qw | ((uint32_t)hs << 8));
  }
  for (size_t e = 0; e < H.entries.size(); ++e) {
    for (int t = 0; t < 4; ++t) {
      int y = H.entries[e][t];
      put16(b + kHtBf16Off + 8 * e + 2 * t, bf16_of_half(y));
      put16(b + kHtA3Off + 8 * e + 2 * t, (uint16_t)(int16_t)(2 * y));
      put16(b + kHtA4Off + 8 * e + 2 * t, (uint16_t)(int16_t)(4 * y));
      put16(b + kHtB4Off + 8 * e + 2 * t, (uint16_t)(kBias + y));
    }
  }
  for (uint32_t i = 0; i < 256; ++i)
    for (int t = 0; t < 8; ++t) put16(b + kR3Off + 16 * i + 2 * t, (uint16_t)(kBias + P[i].y[t]));

  // self-check: decode every index through the tables exactly as the kernels do
  for (uint32_t i = 0; i < kCodebookSize; ++i) {
    int y[8];
    decode_doubled_via_tables(b, i, y);
    for (int t = 0; t < 8; ++t)
      if (y[t] != P[i].y[t]) return false;
  }
  return true;
}

Tables &tables() {
  static Tables T;
  static std::once_flag once;
  std::call_once(once, [] { T.ok = build_tables(T); });
  return T;
}

}  // namespace

// Table walk of glq_tables.h, on the host (used by the self-check above and
// by tests through glq_build_codebook's output).
void decode_doubled_via_tables(const uint8_t *blob, uint32_t i, int *y) {
  auto rd16 = [&](uint32_t off) { uint16_t v; std::memcpy(&v, blob + off, 2); return (uint32_t)v; };
  auto rd32 = [&](uint32_t off) { uint32_t v; std::memcpy(&v, blob + off, 4); return v; };
  uint32_t ip = (i - 1u) & 0xFFFFu;
  uint32_t e = rd16(kCtOff + 2 * (ip >> 4));
  uint32_t low = ip & 15u;
  uint32_t rec = (e >> 5) + (low >> (e & 31u));
  const uint32_t w0 = rd32(kOtOff + 8 * rec), w1 = rd32(kOtOff + 8 * rec + 4);
  const uint32_t r_lo = w0 & 31u, lo_off = w0 >> 8, qw = w1 & 31u;
  const uint32_t hi_off = (uint32_t)((int32_t)w1 >> 8);
  uint32_t jlo = ip & ((1u << r_lo) - 1u);
  uint32_t lo_addr = lo_off + 8u * jlo;
  uint32_t qsrc = qw ? (ip & ((1u << qw) - 1u)) : 0u;
  uint32_t q = (uint32_t)__builtin_popcount(qsrc) & 1u;
  uint32_t hi_addr = hi_off + 8u * (ip >> r_lo) + 64u * q;
  for (int t = 0; t < 4; ++t) {
    y[t] = (int16_t)rd16(kHtA3Off + lo_addr + 2 * t) / 2;
    y[4 + t] = (int16_t)rd16(kHtA3Off + hi_addr + 2 * t) / 2;
  }
}

const int8_t *codebook_doubled() {
  Tables &T = tables();
  return T.ok ? T.flat.data() : nullptr;
}

const uint8_t *device_blob() {
  Tables &T = tables();
  return T.ok ? T.blob.data() : nullptr;
}

}  // namespace glq

extern "C" int glq_build_codebook(int32_t form, void *out, size_t out_bytes, size_t *needed) {
  size_t sz;
  if (form == GLQ_CB_INT8_2X) sz = (size_t)glq::kCodebookSize * 8;
  else if (form == GLQ_CB_DEVICE) sz = glq::kBlobBytes;
  else return GLQ_ERR_ARG;
  if (needed) *needed = sz;
  if (!out) return GLQ_OK;
  if (out_bytes < sz) return GLQ_ERR_WORKSPACE;
  const void *src = form == GLQ_CB_INT8_2X ? (const void *)glq::codebook_doubled()
                                           : (const void *)glq::device_blob();
  if (!src) return GLQ_ERR_UNSUPPORTED;   // table construction failed its self-check
  std::memcpy(out, src, sz);
  return GLQ_OK;
}

extern "C" const char *glq_status_string(int status) {
  switch (status) {
    case GLQ_OK: return "ok";
    case GLQ_ERR_ARG: return "invalid argument";
    case GLQ_ERR_UNSUPPORTED: return "unsupported shape or configuration";
    case GLQ_ERR_HIP: return "HIP runtime or launch error";
    case GLQ_ERR_WORKSPACE: return "workspace or output buffer too small";
    default: return "unknown status";
  }
}

extern "C" uint32_t glq_version(void) { return glq::kFormatVersion; }
