// glq_codebook.cpp -- the E8 codebook in the stated order and its decode tables.
//
// "glq 0.1.1" (PyPI), "How it works", item 1: the codebook holds 65,536
// vectors from the first 7 shells of E8. Format choices the page leaves open:
// standard coordinates (all integer or all half-integer, even sum), the origin
// counted as shell 0, and the order ascending on
//   (|x|^2, -orbit size, max|x_i|, |x| lexicographic, sign counter j)
// with orbit = points sharing |x| (2^nnz points when integer, 128 when
// half-integer), j over the nonzero coordinates in order (integer points) or
// over x1, x2, x3, x5, .., x8 (half-integer points, the sign of x4 fixed by
// the even-sum rule). Format 3 of the tables (glq_tables.h).
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
    static const int coord[7] = {0, 1, 2, 4, 5, 6, 7};   // bit -> coordinate; x4 by parity
    for (int b = 0; b < 7; ++b) if (y[coord[b]] < 0) p.j |= 1u << b;
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

uint16_t bf16_of_half(int y) {  // bf16 bits of y / 2 (exact: |y| <= 6)
  float f = 0.5f * (float)y;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

struct Tables {
  std::vector<Point> pts;
  std::vector<uint8_t> blob;      // GLQ_CB_DEVICE
  std::vector<int8_t> flat;       // GLQ_CB_INT8_2X
  bool ok = false;
};

typedef std::array<int, 4> Half;  // doubled coordinates of 4 consecutive coordinates

// The half-vector table: blocks appended in order, and an index of every
// run of 1, 2 or 4 consecutive entries (content -> first position), so that
// the record of a chunk points into an existing block whenever one holds
// the run it needs.
struct HalfTable {
  std::vector<Half> entries;
  std::map<std::vector<int>, std::vector<uint32_t>> runs;    // content -> positions, increasing
  std::map<std::vector<int>, uint32_t> aligned_runs;         // first position with start % 4 == 0
  std::map<std::pair<int, std::vector<int>>, uint32_t> blocks;  // (kind, |pattern|) -> first entry

  static std::vector<int> key(const std::vector<Half> &r) {
    std::vector<int> k;
    for (const Half &h : r) k.insert(k.end(), h.begin(), h.end());
    return k;
  }
  void index_from(size_t first) {
    for (size_t p = first >= 3 ? first - 3 : 0; p < entries.size(); ++p)
      for (size_t len : {1u, 2u, 4u}) {
        if (p + len > entries.size()) continue;
        std::vector<Half> r(entries.begin() + p, entries.begin() + p + len);
        auto k = key(r);
        auto &v = runs[k];
        if (v.empty() || v.back() < p) v.push_back((uint32_t)p);
        if (p % 4 == 0) aligned_runs.emplace(k, (uint32_t)p);
      }
  }
  uint32_t append(const std::vector<Half> &r) {    // at a multiple of 4
    while (entries.size() % 4) entries.push_back(Half{0, 0, 0, 0});
    const size_t first = entries.size();
    entries.insert(entries.end(), r.begin(), r.end());
    index_from(first);
    return (uint32_t)first;
  }
  uint32_t find_aligned(const std::vector<Half> &r) {
    auto it = aligned_runs.find(key(r));
    return it != aligned_runs.end() ? it->second : append(r);
  }
  uint32_t find_from(const std::vector<Half> &r, uint32_t min_pos) {   // first position >= min_pos
    auto it = runs.find(key(r));
    if (it != runs.end())
      for (uint32_t p : it->second)
        if (p >= min_pos) return p;
    return append(r);
  }
  // every sign pattern of the nonzero coordinates of |a|, coordinate r of
  // the nonzeros negative iff bit r of the entry number is set
  void natural_block(const Half &a) {
    const auto bk = std::make_pair(0, std::vector<int>(a.begin(), a.end()));
    if (blocks.count(bk)) return;
    int pos[4], nnz = 0;
    for (int t = 0; t < 4; ++t) if (a[t]) pos[nnz++] = t;
    std::vector<Half> blk;
    for (uint32_t sg = 0; sg < (1u << nnz); ++sg) {
      Half e = a;
      for (int r = 0; r < nnz; ++r) if (sg >> r & 1) e[pos[r]] = -e[pos[r]];
      blk.push_back(e);
    }
    blocks[bk] = append(blk);
  }
  // half-integer low halves: entry (q << 3) | j3, the signs of x1..x3 from
  // j3 and the sign of x4 negative iff q xor parity(j3)
  void q_block(const Half &a) {
    const auto bk = std::make_pair(1, std::vector<int>(a.begin(), a.end()));
    if (blocks.count(bk)) return;
    std::vector<Half> blk;
    for (uint32_t e = 0; e < 16; ++e) {
      uint32_t q = e >> 3, j3 = e & 7;
      Half v = a;
      for (int t = 0; t < 3; ++t) if (j3 >> t & 1) v[t] = -v[t];
      if ((q ^ j3 ^ (j3 >> 1) ^ (j3 >> 2)) & 1) v[3] = -v[3];
      blk.push_back(v);
    }
    blocks[bk] = append(blk);
  }
};

void put16(uint8_t *p, uint16_t v) { std::memcpy(p, &v, 2); }
void put32(uint8_t *p, uint32_t v) { std::memcpy(p, &v, 4); }

Half lo_half(const Point &p) { return Half{p.y[0], p.y[1], p.y[2], p.y[3]}; }
Half hi_half(const Point &p) { return Half{p.y[4], p.y[5], p.y[6], p.y[7]}; }

bool build_tables(Tables &T) {
  T.pts = build_points();
  const auto &P = T.pts;

  // flat form
  T.flat.resize(kCodebookSize * 8);
  for (uint32_t i = 0; i < kCodebookSize; ++i)
    for (int t = 0; t < 8; ++t) T.flat[i * 8 + t] = P[i].y[t];

  // Blocks first (the zero half at entry 0): the natural sign blocks of
  // every integer half pattern and of every half-integer high half, and the
  // parity blocks of the half-integer low halves; the chunks' runs are then
  // found inside them.
  HalfTable H;
  H.append({Half{0, 0, 0, 0}});
  for (uint32_t i = 0; i < kCodebookSize; ++i) {
    Half lo = lo_half(P[i]), hi = hi_half(P[i]);
    for (int t = 0; t < 4; ++t) { lo[t] = std::abs(lo[t]); hi[t] = std::abs(hi[t]); }
    if (P[i].y[0] & 1) H.q_block(lo);
    else H.natural_block(lo);
    H.natural_block(hi);
  }

  std::vector<uint32_t> rt(kChunks);
  for (uint32_t c = 0; c < kChunks; ++c) {
    Half L[4], Hh[4];
    for (uint32_t m = 0; m < 4; ++m) {
      const uint32_t i = (4 * c + m + 1) & 0xFFFFu;
      L[m] = lo_half(P[i]);
      Hh[m] = hi_half(P[i]);
    }
    // low half: the smallest window width whose 2^t values repeat across the chunk
    uint32_t t_lo = 2;
    if (L[0] == L[1] && L[0] == L[2] && L[0] == L[3]) t_lo = 0;
    else if (L[0] == L[2] && L[1] == L[3]) t_lo = 1;
    // high half: the largest window offset the chunk allows
    uint32_t Toff = 0;
    if (Hh[0] == Hh[1] && Hh[0] == Hh[2] && Hh[0] == Hh[3]) Toff = 2;
    else if (Hh[0] == Hh[1] && Hh[2] == Hh[3]) Toff = 1;
    std::vector<Half> lrun(L, L + (1u << t_lo));
    const uint32_t lo_entry = H.find_aligned(lrun);
    std::vector<Half> hrun;
    if (Toff == 2) hrun = {Hh[0]};
    else if (Toff == 1) hrun = {Hh[0], Hh[2]};
    else hrun = {Hh[0], Hh[1], Hh[2], Hh[3]};
    // the window (i' >> T) & 3 also covers bits of i' that are constant in
    // the chunk: subtract their value at m = 0
    const uint32_t base_off = ((4 * c) >> Toff) & 3u;
    const uint32_t hrun_entry = H.find_from(hrun, base_off);
    const uint32_t hi_entry = hrun_entry - base_off;
    if (lo_entry % 4 || 8 * lo_entry >= 65536 || hi_entry >= kMaxHalves) return false;
    rt[c] = rec_pack(t_lo, 8 * lo_entry, Toff, hi_entry);
  }
  if (H.entries.size() > kMaxHalves) return false;

  // blob
  T.blob.assign(kBlobBytes, 0);
  uint8_t *b = T.blob.data();
  put32(b + 0, kMagic0);
  put32(b + 4, kFormatVersion);
  put32(b + 8, (uint32_t)H.entries.size());
  for (uint32_t c = 0; c < kChunks; ++c) put32(b + kRtOff + 4 * c, rt[c]);
  for (size_t e = 0; e < H.entries.size(); ++e) {
    for (int t = 0; t < 4; ++t) {
      int y = H.entries[e][t];
      put16(b + kHtBf16Off + 8 * e + 2 * t, bf16_of_half(y));
      put16(b + kHtTOff + 8 * e + 2 * t, (uint16_t)((kHtBase + (uint32_t)y) & 0xFFFFu));
    }
  }
  for (uint32_t i = 0; i < 256; ++i)
    for (int t = 0; t < 8; ++t) put16(b + kR3Off + 16 * i + 2 * t, (uint16_t)((kR3Base + (uint32_t)P[i].y[t]) & 0xFFFFu));

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
  const uint32_t ip = (i - 1u) & 0xFFFFu;
  const uint32_t rec = rd32(kRtOff + 4 * (ip >> 2));
  const uint32_t t_lo = rec & 31u, wh = rec >> 16;
  const uint32_t lo_byte = (rec & 0xFFE0u) + 8u * (ip & ((1u << t_lo) - 1u));
  const uint32_t hi_byte = (wh >> 2) + 8u * ((ip >> (wh & 31u)) & 3u);
  for (int t = 0; t < 4; ++t) {
    y[t] = (int)(int16_t)(uint16_t)(rd16(kHtTOff + lo_byte + 2 * t) - kHtBase);
    y[4 + t] = (int)(int16_t)(uint16_t)(rd16(kHtTOff + hi_byte + 2 * t) - kHtBase);
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
