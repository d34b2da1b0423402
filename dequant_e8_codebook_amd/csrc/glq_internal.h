// glq_internal.h -- declarations shared by the library's own source files.
#pragma once
#include <stdint.h>

namespace glq {

// The codebook as doubled coordinates y = 2x, int8 [65536][8], or NULL if
// the tables failed their construction self-check.
const int8_t *codebook_doubled();

// The GLQ_CB_DEVICE blob (kBlobBytes bytes), or NULL.
const uint8_t *device_blob();

// Decode index i through the chunk/record/half tables of a GLQ_CB_DEVICE blob
// (host version of the kernels' table walk) into doubled coordinates y[8].
void decode_doubled_via_tables(const uint8_t *blob, uint32_t i, int *y);

}  // namespace glq
