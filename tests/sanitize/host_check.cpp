// host_check.cpp -- drives the library's CPU entry points (codebook tables,
// both encoders, the entropy coder and its decode tables) on small layers,
// built together with the host sources under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitize_host.py). It checks what
// needs no oracle: the codebook's shape and order invariants, thread-count
// determinism of every encoder, the error paths, and that every block of an
// entropy-coded stream decodes (rANS, the format in glq.h) with all its
// words consumed and its lanes back at the start state.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "glq.h"

static int g_fail = 0;
#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

static std::vector<float> weights(int64_t n, int64_t k, unsigned seed) {
  std::mt19937 g(seed);
  std::student_t_distribution<float> t(5.0f);
  std::vector<float> w((size_t)(n * k));
  for (auto &v : w) v = 0.02f * t(g) / std::sqrt(5.0f / 3.0f);
  return w;
}

static std::vector<int8_t> signs(int64_t len, unsigned seed) {
  std::mt19937 g(seed);
  std::vector<int8_t> s((size_t)len);
  for (auto &v : s) v = (g() & 1) ? 1 : -1;
  return s;
}

static void codebook_checks() {
  size_t need = 0;
  CHECK(glq_build_codebook(GLQ_CB_INT8_2X, nullptr, 0, &need) == GLQ_OK && need == 65536 * 8);
  std::vector<int8_t> cb(need);
  CHECK(glq_build_codebook(GLQ_CB_INT8_2X, cb.data(), cb.size(), nullptr) == GLQ_OK);
  int prev = -1, bad = 0;
  for (int i = 0; i < 65536; ++i) {
    int n4 = 0, sum = 0, odd = cb[8 * i] & 1;
    for (int t = 0; t < 8; ++t) {
      n4 += cb[8 * i + t] * cb[8 * i + t];
      sum += cb[8 * i + t];
      bad += (cb[8 * i + t] & 1) != odd;
    }
    bad += ((sum % 4) + 4) % 4 != 0;
    bad += n4 < prev;
    prev = n4;
  }
  CHECK(bad == 0);
  size_t dn = 0;
  CHECK(glq_build_codebook(GLQ_CB_DEVICE, nullptr, 0, &dn) == GLQ_OK && dn > 65536);
  std::vector<uint8_t> blob(dn);
  CHECK(glq_build_codebook(GLQ_CB_DEVICE, blob.data(), blob.size(), nullptr) == GLQ_OK);
  CHECK(glq_build_codebook(GLQ_CB_DEVICE, blob.data(), 16, nullptr) == GLQ_ERR_WORKSPACE);
  CHECK(glq_build_codebook(9, nullptr, 0, &dn) == GLQ_ERR_ARG);
  CHECK(glq_version() == 0x00030000u);
}

static void encoder_checks() {
  const int64_t n = 24, k = 96;
  const auto w = weights(n, k, 11);
  const auto sn = signs(n, 12), sk = signs(k, 13);
  for (int bpw = 2; bpw <= 4; ++bpw) {
    const size_t g = (size_t)(n * k / 8), i2b = bpw == 3 ? 1 : 2;
    std::vector<uint16_t> a1(g), b1(g);
    std::vector<uint8_t> a2(g * i2b), b2(g * i2b);
    std::vector<float> rs(n);
    float s1 = 0, s2 = 0;
    void *p2a = bpw > 2 ? (void *)a2.data() : nullptr, *p2b = bpw > 2 ? (void *)b2.data() : nullptr;
    CHECK(glq_encode_ref(w.data(), n, k, bpw, sn.data(), sk.data(), 0.0f, &s1, a1.data(), p2a, 1, nullptr) == GLQ_OK);
    CHECK(glq_encode_ref(w.data(), n, k, bpw, sn.data(), sk.data(), 0.0f, &s2, b1.data(), p2b, 3, nullptr) == GLQ_OK);
    CHECK(s1 == s2 && s1 > 0 && a1 == b1 && a2 == b2);
    CHECK(glq_encode_ref(w.data(), n, k, bpw, sn.data(), sk.data(), 0.0f, &s2, b1.data(), p2b, 2, rs.data()) == GLQ_OK);
    for (float r : rs) CHECK(std::isfinite(r) && r > 0);
    // Hessian of random calibration rows (symmetric positive definite)
    std::vector<double> h((size_t)(k * k), 0.0);
    std::mt19937 gen(7 + bpw);
    std::normal_distribution<double> nd;
    for (int r = 0; r < 3 * k; ++r) {
      std::vector<double> x(k);
      for (auto &v : x) v = nd(gen);
      for (int64_t a = 0; a < k; ++a)
        for (int64_t b = 0; b < k; ++b) h[a * k + b] += x[a] * x[b] / (3.0 * k);
    }
    CHECK(glq_encode_ldlq(w.data(), n, k, bpw, sn.data(), sk.data(), h.data(), 0.01, 0.0f, &s1, a1.data(), p2a, 1,
                          nullptr) == GLQ_OK);
    CHECK(glq_encode_ldlq(w.data(), n, k, bpw, sn.data(), sk.data(), h.data(), 0.01, 0.0f, &s2, b1.data(), p2b, 4,
                          nullptr) == GLQ_OK);
    CHECK(a1 == b1 && a2 == b2);
  }
  std::vector<uint16_t> i1(8);
  CHECK(glq_encode_ref(w.data(), n, 60, 2, sn.data(), sk.data(), 0.0f, nullptr, i1.data(), nullptr, 1, nullptr) ==
        GLQ_ERR_ARG);
  CHECK(glq_encode_ref(nullptr, n, k, 2, sn.data(), sk.data(), 0.0f, nullptr, i1.data(), nullptr, 1, nullptr) ==
        GLQ_ERR_ARG);
  CHECK(glq_encode_ref(w.data(), n, k, 5, sn.data(), sk.data(), 0.0f, nullptr, i1.data(), nullptr, 1, nullptr) ==
        GLQ_ERR_ARG);
  CHECK(glq_encode_ldlq(w.data(), n, k, 2, sn.data(), sk.data(), nullptr, 0.01, 0.0f, nullptr, i1.data(), nullptr, 1,
                        nullptr) == GLQ_ERR_ARG);
}

// rANS decode of one block (11-bit precision, 16-bit words), the format of
// glq.h; returns the number of words used, or -1 on an inconsistency
static long decode_block(const glq_ep_model &m, long ngroups, const uint32_t *st, const uint16_t *words, long nw) {
  uint32_t x[64];
  std::memcpy(x, st, sizeof x);
  std::vector<int32_t> z0(64);
  long pos = 0;
  for (long p = 0; p * 64 < ngroups; ++p) {
    for (int c = 0; c < 8; ++c) {
      for (int l = 0; l < 64 && p * 64 + l < ngroups; ++l) {
        const int tab = c == 0 ? 0 : (c < 7 ? 1 : 3) + (z0[l] & 1);
        if (m.nsym[tab] <= 0) return -1;
        const uint32_t slot = x[l] & 2047u;
        uint32_t cum = 0;
        int s = 0;
        while (s < m.nsym[tab] && cum + m.freq[tab][s] <= slot) cum += m.freq[tab][s++];
        if (s >= m.nsym[tab]) return -1;
        x[l] = m.freq[tab][s] * (x[l] >> 11) + slot - cum;
        if (c == 0) z0[l] = m.vmin[0] + s;
      }
      for (int l = 0; l < 64 && p * 64 + l < ngroups; ++l)
        if (x[l] < (1u << 16)) {
          if (pos >= nw) return -1;
          x[l] = (x[l] << 16) | words[pos++];
        }
    }
  }
  for (int l = 0; l < 64; ++l)
    if (x[l] != (1u << 16)) return -1;
  return pos;
}

static void ep_checks() {
  const int64_t n = 20, k = 136;
  const auto w = weights(n, k, 21);
  const auto sn = signs(n, 22), sk = signs(k, 23);
  for (int lg : {1, 3}) {
    const long groups = (long)(n * k / 8), nb = (groups + 64 * lg - 1) / (64 * lg);
    std::vector<float> rs(n), rs2(n);
    glq_ep_model m{}, m2{};
    std::vector<uint32_t> st((size_t)nb * 64), st2((size_t)nb * 64), off(nb + 1), off2(nb + 1);
    std::vector<uint16_t> words((size_t)(n * k)), words2((size_t)(n * k));
    int64_t nw = 0, nw2 = 0;
    CHECK(glq_ep_encode(w.data(), n, k, sn.data(), sk.data(), 0.3f, lg, 1, rs.data(), &m, st.data(), off.data(),
                        words.data(), (int64_t)words.size(), &nw) == GLQ_OK);
    CHECK(glq_ep_encode(w.data(), n, k, sn.data(), sk.data(), 0.3f, lg, 3, rs2.data(), &m2, st2.data(), off2.data(),
                        words2.data(), (int64_t)words2.size(), &nw2) == GLQ_OK);
    CHECK(nw == nw2 && st == st2 && off == off2 && rs == rs2 && std::memcmp(&m, &m2, sizeof m) == 0);
    CHECK(std::equal(words.begin(), words.begin() + nw, words2.begin()));
    for (long b = 0; b < nb; ++b) {
      const long ng = std::min<long>(64L * lg, groups - 64L * lg * b);
      const long used = decode_block(m, ng, &st[64 * b], &words[off[b]], (long)(off[b + 1] - off[b]));
      CHECK(used == (long)(off[b + 1] - off[b]));
    }
    std::vector<uint8_t> lut(GLQ_EP_LUT_BYTES);
    CHECK(glq_ep_build_lut(&m, lut.data(), lut.size()) == GLQ_OK);
    CHECK(glq_ep_build_lut(&m, lut.data(), 10) == GLQ_ERR_ARG);
    int64_t need = 0;
    CHECK(glq_ep_encode(w.data(), n, k, sn.data(), sk.data(), 0.3f, lg, 1, rs.data(), &m, st.data(), off.data(),
                        words.data(), 1, &need) == GLQ_ERR_WORKSPACE);
    CHECK(need == nw);
  }
  glq_ep_model m{};
  std::vector<float> rs(n);
  std::vector<uint32_t> st(64 * 64), off(65);
  std::vector<uint16_t> words((size_t)(n * k));
  int64_t nw = 0;
  CHECK(glq_ep_encode(w.data(), n, k, sn.data(), sk.data(), 0.0f, 1, 1, rs.data(), &m, st.data(), off.data(),
                      words.data(), (int64_t)words.size(), &nw) == GLQ_ERR_ARG);
  CHECK(glq_ep_encode(w.data(), n, k, sn.data(), sk.data(), 0.002f, 1, 1, rs.data(), &m, st.data(), off.data(),
                      words.data(), (int64_t)words.size(), &nw) == GLQ_ERR_UNSUPPORTED);
}

int main() {
  codebook_checks();
  encoder_checks();
  ep_checks();
  CHECK(std::strlen(glq_status_string(GLQ_ERR_HIP)) > 0);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host_check ok\n");
  return 0;
}
