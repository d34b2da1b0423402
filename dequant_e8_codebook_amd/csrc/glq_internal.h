// glq_internal.h -- declarations shared by the library's own source files.
#pragma once
#include <stdint.h>

#include <atomic>
#include <thread>
#include <vector>

namespace glq {

// The codebook as doubled coordinates y = 2x, int8 [65536][8], or NULL if
// the tables failed their construction self-check.
const int8_t *codebook_doubled();

// The GLQ_CB_DEVICE blob (kBlobBytes bytes), or NULL.
const uint8_t *device_blob();

// Decode index i through the record and half-vector tables of a GLQ_CB_DEVICE blob
// (host version of the kernels' table walk) into doubled coordinates y[8].
void decode_doubled_via_tables(const uint8_t *blob, uint32_t i, int *y);

// W~ = U W V^T in float64 for W [n][k]: randomized Hadamard transform of every
// row (signs sign_k, blocks of the largest power of two dividing k), then of
// every column (sign_n); out is [n][k].
void rotate_weights_f64(const float *w, int64_t n, int64_t k, const int8_t *sign_n,
                        const int8_t *sign_k, int nthreads, double *out);

// fn(i) for i in [0, count) on up to nthreads threads (work taken in order)
template <class F>
void parallel_for(int64_t count, int nthreads, F fn) {
  if (nthreads <= 1 || count < 2) {
    for (int64_t i = 0; i < count; ++i) fn(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> th;
  for (int t = 0; t < nthreads; ++t)
    th.emplace_back([&] {
      while (true) {
        int64_t i = next.fetch_add(1);
        if (i >= count) break;
        fn(i);
      }
    });
  for (auto &t : th) t.join();
}

}  // namespace glq
