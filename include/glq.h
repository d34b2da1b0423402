/*
 * glq.h -- C ABI of the E8-lattice-codebook linear layer for MI355X (gfx950).
 *
 * What the library computes (the method of "glq 0.1.1", PyPI project page,
 * section "How it works", items 1-2, and section "Bit widths"):
 *
 *   Every group of 8 consecutive weights of a rotated weight matrix
 *   W~ = U W V^T  [n, k]  is stored as a 16-bit index into a 65,536-entry
 *   E8 lattice codebook C, optionally plus an 8-bit (3 bpw) or 16-bit
 *   (4 bpw) index into a residual codebook, with one global float32 scale s
 *   per layer:   W^[r, 8g:8g+8] = s * ( C[i1] + 2^-k * C_r[i2] ).
 *   U and V are randomized Hadamard transforms: random sign flips followed
 *   by a (block-diagonal) fast Walsh-Hadamard transform, normalised by
 *   1/sqrt(b).  At run time a layer computes
 *
 *       y = U^T ( s W^ ) ( V x )
 *
 *   reconstructing W^ inside the matrix product ("EntroPack" news item:
 *   the GPU fuses symbol decoding and weight reconstruction; storage rate is
 *   kept separate from compute precision).
 *
 * Format decisions the pages leave open (all stated in the library's design
 * notes): standard E8 coordinates; the origin counts as shell 0; codebook
 * order = ascending (|x|^2, -orbit size, max|x_i|, |x| lexicographic, sign
 * counter); C_r = the first 2^8 (3 bpw) or 2^16 (4 bpw) codebook entries
 * with k = 1 (3 bpw) or k = 2 (4 bpw); groups run along k; Sylvester
 * Hadamard in natural order, block b(n) = largest power of two dividing n.
 *
 * Conventions for every call:
 *  - All memory is owned and allocated by the caller. No call allocates or
 *    frees memory, device or host (the CPU encoders allocate host scratch).
 *  - Device pointers are HIP device pointers; "host" marks host pointers.
 *  - Every call returns a glq_status. Arguments are validated before any
 *    launch; no error aborts the process or escapes as an exception.
 *  - GPU calls are asynchronous on the given HIP stream (NULL = default
 *    stream), never synchronise the host, and keep no state between calls:
 *    calls on different streams may run concurrently.
 *  - Layouts are dense row-major with no padding.
 */
#ifndef GLQ_H
#define GLQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GLQ_OK = 0,
    GLQ_ERR_ARG = -1,          /* invalid argument (null pointer, bad size, bad enum) */
    GLQ_ERR_UNSUPPORTED = -2,  /* valid but unsupported shape (e.g. Hadamard block > 16384) */
    GLQ_ERR_HIP = -3,          /* a HIP launch or runtime call failed */
    GLQ_ERR_WORKSPACE = -4     /* workspace missing or smaller than required */
} glq_status;

typedef enum { GLQ_F32 = 0, GLQ_BF16 = 1 } glq_dtype;

/* codebook forms for glq_build_codebook */
enum {
    GLQ_CB_INT8_2X = 0,  /* host table int8 [65536][8] holding 2*C[i] (doubled coordinates) */
    GLQ_CB_DEVICE = 1    /* opaque decode tables; copy the bytes to device memory unchanged */
};

/* flags for glq_fused_linear */
enum {
    GLQ_FLAG_NO_INPUT_RHT = 1u,   /* x is already rotated: use x~ = x */
    GLQ_FLAG_NO_OUTPUT_RHT = 2u   /* return z = s W^ x~ (rotated basis) instead of y = U^T z */
};

/* One compressed linear layer. The struct itself lives in host memory; the
 * pointers in it are device pointers owned by the caller. */
typedef struct {
    int64_t n;                /* out features (rows of W), >= 1 */
    int64_t k;                /* in features, >= 8 and k % 8 == 0 */
    int32_t bpw;              /* 2, 3 or 4 */
    int32_t resid_shift;      /* residual scale 2^-resid_shift: must be 1 at 3 bpw, 2 at 4 bpw; ignored at 2 bpw */
    float scale;              /* the global scale s (finite, > 0) */
    const uint16_t *idx1;     /* [n][k/8] stage-1 codebook indices */
    const void *idx2;         /* [n][k/8] residual indices: uint8 (3 bpw), uint16 (4 bpw), NULL (2 bpw) */
    const int8_t *sign_k;     /* [k] input-side signs, each +1 or -1 */
    const int8_t *sign_n;     /* [n] output-side signs, each +1 or -1 */
    const void *cb;           /* device copy of the GLQ_CB_DEVICE tables */
    const float *row_scale;   /* device float [n] per-row scales, or NULL ("EntroPack" news
                                 item: per-row normalised E8): row r then decodes with the
                                 scale s_r = fl32(scale * row_scale[r]) in place of scale;
                                 each entry finite and > 0 */
} glq_layer;

/*
 * glq_build_codebook -- write the codebook ("glq 0.1.1", "How it works",
 * item 1: 65,536 E8 vectors from the first 7 shells) in the stated order.
 *   form       GLQ_CB_INT8_2X or GLQ_CB_DEVICE
 *   out        host buffer of out_bytes bytes, or NULL to query the size
 *   needed     host; if not NULL receives the size in bytes of the form
 * Returns GLQ_ERR_ARG for an unknown form and GLQ_ERR_WORKSPACE when out is
 * not NULL and out_bytes is too small (nothing is written then).
 */
int glq_build_codebook(int32_t form, void *out, size_t out_bytes, size_t *needed);

/*
 * glq_encode_ref -- CPU encoder ("glq 0.1.1", "How it works", items 1-2;
 * "Bit widths"): W~ = U W V^T in float64, s = fp32(sqrt(mean(W~^2))) unless
 * given, X = W~/s in groups of 8 along k, i1 = nearest codebook entry (float64
 * squared distance, lowest index on ties), and for 3/4 bpw i2 = nearest entry
 * of 2^-k C_r to the residual X - C[i1]. Nearest-neighbour rounding of every
 * group on its own (glq_encode_ldlq adds the page's error feedback).
 *   w          host float [n][k], original (unrotated) basis, finite
 *   sign_n     host int8 [n] (+1/-1),  sign_k  host int8 [k] (+1/-1)
 *   scale_in   > 0: use as s;  <= 0: compute s as above
 *   scale_out  host, receives s (may be NULL)
 *   idx1_out   host uint16 [n][k/8]
 *   idx2_out   host uint8 (3 bpw) / uint16 (4 bpw) [n][k/8]; NULL at 2 bpw
 *   nthreads   worker threads (<= 0: hardware concurrency)
 *   row_scale_out  host float [n], or NULL. When given, every row gets its own
 *              scale ("EntroPack" news item: per-row normalised E8): s_r =
 *              fp32(sqrt(mean_j W~[r,j]^2)) (1 for a zero row) is written to
 *              row_scale_out[r], row r is divided by s_r before the search,
 *              scale_in is ignored and *scale_out receives 1.
 * Returns GLQ_ERR_ARG for bad sizes/bpw, non-finite weights or signs not +-1.
 */
int glq_encode_ref(const float *w, int64_t n, int64_t k, int32_t bpw,
                   const int8_t *sign_n, const int8_t *sign_k,
                   float scale_in, float *scale_out,
                   uint16_t *idx1_out, void *idx2_out, int32_t nthreads,
                   float *row_scale_out);

/*
 * glq_encode_ldlq -- CPU encoder with LDLQ error feedback ("glq 0.1.1", "How
 * it works", item 3: a block LDL decomposition of the Hessian drives a
 * sequential sweep over 8-weight blocks, each block's quantisation error
 * corrects the blocks after it, as in GPTQ; item 2: the Hessian is rotated
 * like the weights). With X = W~/s as in glq_encode_ref:
 *   H~ = V H V^T + damp * mean(diag(V H V^T)) * I
 *   H~ = (I + U) D (I + U)^T, U strictly block upper triangular (blocks of 8)
 *   for j = 0 .. k/8-1, every row:  T_j = X_j + sum_{i<j} (X_i - X^_i) U_ij,
 *                                   X^_j = Q(T_j)
 * with Q the nearest-entry / residual quantiser of glq_encode_ref (float64
 * throughout). Every other argument is as in glq_encode_ref.
 *   hessian    host double [k][k], symmetric positive semi-definite, over the
 *              input features in the original basis (e.g. X^T X / m for
 *              calibration inputs X [m][k]); read only; k <= 16384
 *   damp       >= 0; GPTQ's dampening fraction (0.01 is its default)
 * Host scratch of about 1.5 k^2 doubles plus n k doubles is allocated.
 * Returns GLQ_ERR_ARG as glq_encode_ref does, and also for a NULL or
 * non-finite Hessian, a negative or non-finite damp, or a damped rotated
 * Hessian that is not positive definite; GLQ_ERR_UNSUPPORTED for k > 16384.
 */
int glq_encode_ldlq(const float *w, int64_t n, int64_t k, int32_t bpw,
                    const int8_t *sign_n, const int8_t *sign_k,
                    const double *hessian, double damp,
                    float scale_in, float *scale_out,
                    uint16_t *idx1_out, void *idx2_out, int32_t nthreads,
                    float *row_scale_out);

/*
 * glq_rht_apply -- randomized Hadamard transform along the last axis of a
 * [rows][n] array ("glq 0.1.1", "How it works", item 2), b = largest power of
 * two dividing n (<= 16384), computed in float32:
 *   transpose = 0:  out = (I (x) H_b) diag(signs) in / sqrt(b)   (signs, then FWHT)
 *   transpose = 1:  out = diag(signs) (I (x) H_b) in / sqrt(b)   (FWHT, then signs)
 *   in, out    device, dtype in_dt / out_dt; may be the same buffer when
 *              in_dt == out_dt
 *   signs      device int8 [n]
 * rows == 0 is a successful no-op.
 */
int glq_rht_apply(const void *in, glq_dtype in_dt, void *out, glq_dtype out_dt,
                  int64_t rows, int64_t n, const int8_t *signs,
                  int32_t transpose, void *hip_stream);

/*
 * glq_decode_weights -- expand the index planes into the rotated-basis
 * weights W^ [n][k] (the reconstruction the fused kernels do on the fly):
 * v = C[i1] + 2^-k C_r[i2] exactly, w = fl32(s * v) (one float32 multiply;
 * s = s_r of the row when L->row_scale is given), bf16 output =
 * round-to-nearest-even of w.
 *   w_out      device [n][k] of out_dt
 */
int glq_decode_weights(const glq_layer *L, void *w_out, glq_dtype out_dt, void *hip_stream);

/* Bytes of device workspace glq_fused_linear needs for m rows (any dtype, any
 * flags), including the control words at its start (GLQ_WS_CTRL_BYTES). */
#define GLQ_WS_CTRL_BYTES 4352
size_t glq_fused_linear_workspace(const glq_layer *L, int64_t m);

/*
 * glq_fused_linear -- y = U^T (s W^) (V x) for x [m][k], y [m][n], with the
 * weights reconstructed inside the product and never written to memory.
 *   x_dt = GLQ_F32:  float32 path (float32 x~, exact float32 weights, float32
 *                    accumulation)
 *   x_dt = GLQ_BF16: bf16 matrix-core path (x~ rounded to bf16, weights exact
 *                    in bf16, float32 accumulation, scale in the epilogue)
 *   y_dt             GLQ_F32 or GLQ_BF16 (round-to-nearest-even)
 *   workspace        device, >= glq_fused_linear_workspace(L, m) bytes, 256-byte aligned.
 *                    Its first GLQ_WS_CTRL_BYTES bytes are control words
 *                    (completion counters of the single-launch layer used at
 *                    small m, and the tile counters of the k-split GEMM used
 *                    for long rows with fewer output tiles than CUs): they
 *                    must be zero before the first call with a
 *                    workspace, every call that returns GLQ_OK (and whose
 *                    kernels complete) leaves them zero, and calls that run
 *                    concurrently need separate workspaces. After a call that
 *                    returned GLQ_ERR_HIP, or whose kernels were aborted, the
 *                    caller must zero those GLQ_WS_CTRL_BYTES again before the
 *                    workspace's next use. The rest is scratch.
 *   flags            GLQ_FLAG_* (0 = the full layer)
 * m == 0 is a successful no-op. x and y must not overlap the workspace.
 */
int glq_fused_linear(const glq_layer *L, const void *x, glq_dtype x_dt, int64_t m,
                     void *y, glq_dtype y_dt, void *workspace, size_t ws_bytes,
                     uint32_t flags, void *hip_stream);

/*
 * glq_fused_linear_noalloc -- glq_fused_linear with no workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, layouts, results and errors as glq_fused_linear (the same
 * kernels run). Its scratch is a static device array of
 * GLQ_STATIC_WS_BYTES bytes per GPU, created with the library's code object
 * and held until the process ends; the call itself allocates nothing. The
 * first call on a device looks up that GPU's copy and clears its control
 * words with a small kernel on the given stream (also after a call that
 * returned GLQ_ERR_HIP). All calls on one GPU share the array: calls that
 * overlap in time on one GPU (different streams, or host threads) race and
 * give undefined results; serialise them.
 * Returns GLQ_ERR_WORKSPACE (glq_last_error names both sizes) when the layer
 * at m rows needs more than GLQ_STATIC_WS_BYTES, that is when
 * glq_fused_linear_workspace(L, m) > GLQ_STATIC_WS_BYTES (about m (k + n)
 * 4 bytes: e.g. m <= 16 rows at any n, k <= 16384, or ~1000 rows of a
 * 4096 x 4096 layer); GLQ_ERR_UNSUPPORTED for a device index >= 64.
 */
#define GLQ_STATIC_WS_BYTES (32u << 20)
int glq_fused_linear_noalloc(const glq_layer *L, const void *x, glq_dtype x_dt, int64_t m,
                             void *y, glq_dtype y_dt, uint32_t flags, void *hip_stream);

/* ------------------------------------------------------------------------
 * Entropy-coded E8 lattice layers ("Transformers Proposes EntroPack
 * Integration ...", first two paragraphs: per-row normalised E8 lattice
 * quantisation, a conditional probability model and entropy coding give any
 * non-integer average storage rate; the coded coordinates are cut into
 * independently decodable blocks; the GPU decodes the symbols and rebuilds
 * the weights in one fused step; actual_bpp counts metadata). The page gives
 * no formulas; the format below is this library's reading of it.
 *
 *  quantiser   s_r = fp32(sqrt(mean_j W~[r,j]^2)) per row (W~ = U W V^T as in
 *              glq_encode_ref), z = 2 * (nearest point of the whole E8
 *              lattice to (W~[r] / s_r) / step), one 8-vector per group of 8
 *              inputs. Decoded weight fl32(fl32(step * s_r) * (z / 2)); bf16 =
 *              round to nearest even of it.
 *  symbols     per group: z_1 (table 0; b = z_1 mod 2), (z_c - b)/2 for
 *              c = 2..7 (table 1 + b), (z_8 - t)/4 with t = -(z_1+..+z_7) mod 4
 *              (table 3 + b). Static per-layer frequencies, 11-bit precision.
 *  coder       rANS, 32-bit state in [2^16, 2^32), 16-bit words.
 *  blocks      groups in row-major order (row r, group q), 64 * lane_groups
 *              per block (the last may be short); group j of a block belongs to
 *              lane j mod 64; the 64 lanes decode in lockstep and take the
 *              words of one step from the block's stream in lane order.
 * ---------------------------------------------------------------------- */
#define GLQ_EP_LANES 64
#define GLQ_EP_TABLES 5
#define GLQ_EP_MAX_SYMS 256
#define GLQ_EP_LUT_BYTES (64 + GLQ_EP_TABLES * 2048 * 4)

/* The probability model: per table the value of symbol 0, the span of
 * values (0 = table unused) and the frequencies (sum 2048 when used). */
typedef struct {
    int32_t vmin[GLQ_EP_TABLES];
    int32_t nsym[GLQ_EP_TABLES];
    uint16_t freq[GLQ_EP_TABLES][GLQ_EP_MAX_SYMS];
} glq_ep_model;

/* One coded layer on the device. nblocks = ceil(n k / 8 / (64 lane_groups)). */
typedef struct {
    int64_t n, k;                /* out, in features; k % 8 == 0; n k / 8 < 2^31 */
    int32_t lane_groups;         /* groups per lane, >= 1 */
    float   step;                /* quantiser step (> 0) */
    const float    *row_scale;   /* device float [n]: s_r */
    const uint32_t *states;      /* device [nblocks][64]: rANS start state of every lane */
    const uint32_t *offsets;     /* device [nblocks + 1]: first word of each block's stream */
    const uint16_t *words;       /* device, 16-byte aligned, [nwords rounded up to a multiple of 8, at least 8] */
    int64_t nwords;              /* offsets[nblocks] */
    const void     *lut;         /* device, GLQ_EP_LUT_BYTES from glq_ep_build_lut */
    const int8_t   *sign_k, *sign_n;  /* device [k], [n] (+1/-1); used by glq_ep_fused_linear only */
} glq_ep_layer;

/*
 * glq_ep_encode -- CPU encoder of the format above (float64 arithmetic; the
 * nearest lattice point by Conway & Sloane's decoder: coordinates rounded half
 * to even, the parity fixed on the first coordinate with the largest
 * rounding error, the integer coset kept on equal distances).
 *   w, sign_n, sign_k   as in glq_encode_ref
 *   step                > 0, finite: the rate control (smaller = more bits)
 *   lane_groups         >= 1 (32 keeps the per-lane state near 2% of the stream
 *                       at 3-4 bits per weight)
 *   row_scale_out       host float [n]
 *   model_out           host
 *   states_out          host uint32 [nblocks][64]
 *   offsets_out         host uint32 [nblocks + 1]
 *   words_out           host uint16 [words_capacity]; n k words always suffice
 *   words_written       host, receives the number of words
 * Returns GLQ_ERR_ARG for bad arguments, GLQ_ERR_UNSUPPORTED when a table
 * would span more than 256 values (step too small for the weights) or
 * n k / 8 >= 2^31, GLQ_ERR_WORKSPACE when words_capacity is too small
 * (*words_written then holds the number needed).
 */
int glq_ep_encode(const float *w, int64_t n, int64_t k, const int8_t *sign_n, const int8_t *sign_k,
                  float step, int32_t lane_groups, int32_t nthreads,
                  float *row_scale_out, glq_ep_model *model_out, uint32_t *states_out,
                  uint32_t *offsets_out, uint16_t *words_out, int64_t words_capacity,
                  int64_t *words_written);

/*
 * glq_ep_build_lut -- CPU: the decode table blob of a model (GLQ_EP_LUT_BYTES;
 * copy it to device memory unchanged): the five vmin values, then per table
 * 2048 slots, slot -> symbol | frequency << 8 | (slot - cumulative) << 20.
 * Returns GLQ_ERR_ARG for a model whose used tables do not sum to 2048 or a
 * buffer smaller than GLQ_EP_LUT_BYTES.
 */
int glq_ep_build_lut(const glq_ep_model *model, void *lut_out, size_t lut_bytes);

/*
 * glq_ep_decode_weights -- GPU: fused symbol decode and weight reconstruction
 * of every group, w_out [n][k] row-major in the rotated basis, bf16 or float32
 * (16-byte aligned). One wave per block. The words buffer is read 16 bytes at
 * a time: it must be 16-byte aligned and hold nwords entries rounded up to a
 * multiple of 8 (at least 8); reads are clamped to it, so a corrupt stream
 * gives wrong weights, never an access outside the buffers.
 */
int glq_ep_decode_weights(const glq_ep_layer *L, void *w_out, glq_dtype out_dt, void *hip_stream);

/*
 * glq_ep_fused_linear -- the layer on an entropy-coded weight set:
 * y = U^T (W^ (V x)) with W^ as glq_ep_decode_weights gives it (the weights
 * carry their row scales and step). x~ = V x is rounded to bf16. Then:
 *   m = 1, k >= 512 and a block's rows fit the kernel's LDS row sums
 *     (always for lane_groups <= 128): the decode is fused into the product.
 *     Each group's 8 weights are reconstructed in float32 (exactly as the
 *     decode gives them) and multiplied into z = x~ W^T with float32 sums;
 *     W^ is never stored. Sums from different blocks of groups meet in
 *     float32 atomic adds, so z (and y) can differ between calls in the
 *     last bits.
 *   otherwise: W^ is decoded to bf16 in the workspace and z = x~ W^T runs on
 *     bf16 matrix cores with float32 accumulation (z kept in float32, or bf16
 *     for bf16 y when m > 16).
 * Then y = U^T z. Flags, dtypes and m as in glq_fused_linear; with
 * GLQ_FLAG_NO_INPUT_RHT, x must be bf16 and 16-byte aligned
 * (GLQ_ERR_UNSUPPORTED otherwise).
 *   workspace   device, >= glq_ep_fused_linear_workspace(L, m) bytes (2 n k,
 *               unless the fused batch-1 product applies, + 2 m k + 4 m n,
 *               each part 256-byte aligned), 256-byte aligned; owned by the
 *               caller, overwritten on every call, and must not overlap x or y
 *               (calls that share one workspace on concurrent streams race)
 */
size_t glq_ep_fused_linear_workspace(const glq_ep_layer *L, int64_t m);
int glq_ep_fused_linear(const glq_ep_layer *L, const void *x, glq_dtype x_dt, int64_t m, void *y,
                        glq_dtype y_dt, void *workspace, size_t ws_bytes, uint32_t flags, void *hip_stream);

/* Static text for a status code. */
const char *glq_status_string(int status);

/* Text of the last HIP failure seen by a GPU call on this thread ("" if none):
 * the HIP call or launch, its error string and code. Static storage, valid
 * until the next GPU call on the same thread. */
const char *glq_last_error(void);

/* Library and codebook-format version, e.g. 0x00030000. */
uint32_t glq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GLQ_H */
