/*
 * jolt.h -- C ABI of the JoLT KV-cache codec hot path on AMD Instinct MI355X
 * (CDNA4, gfx950).
 *
 * Method: "A JoLT for the KV Cache: Near-Lossless KV Cache Compression via
 * Joint Tucker and JL-Residual Allocation for LLMs" (arXiv 2607.12550v2),
 * abstract: each layer's K or V cache is a third-order tensor over heads,
 * tokens and features; a partial Tucker decomposition compresses only the
 * token and feature axes; the energy the truncation drops comes back as a
 * residual that is rotated by a seeded random orthogonal matrix and then
 * quantized to few bits; one Lagrangian dual
 * allocates Tucker ranks and residual bit-widths per layer group, separately
 * for keys and values, under one byte budget; FlashJoLT computes the factors
 * with a randomized SVD.
 *
 * Conventions for every entry point
 *   - Tensors are X[H][T][D] row-major (D fastest), bf16 or fp32, in device
 *     memory.  D must be 128 (the head dimension of the models the method is
 *     evaluated on); T >= 1, H >= 1.
 *   - Every device buffer (inputs, outputs, compressed records, workspaces)
 *     is allocated and owned by the caller.  The library allocates no device
 *     memory (the profiling hooks below excepted) and keeps no device state
 *     between calls.  On the host it keeps a per-device pool of auxiliary HIP
 *     streams (non-blocking, default priority), guarded by a mutex: a call
 *     that forks work onto a second stream leases one for its duration, so
 *     two calls in flight never share an auxiliary stream, and every event a
 *     call records is created for that call alone.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously unless the entry point says it synchronizes.
 *   - Arguments are validated before any work is enqueued; on error nothing
 *     is enqueued and no output is written.  No C++ exception crosses the ABI.
 *   - A device-side fault surfaces as JOLT_EHIP from the next call that
 *     synchronizes.  Calls on distinct streams with distinct workspaces and
 *     output buffers may run concurrently from several host threads (the
 *     profiling and debug hooks excepted).
 */
#ifndef JOLT_H
#define JOLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JOLT_OK = 0,
  JOLT_EINVAL = -1,     /* bad argument (shape, dtype, choice, NULL pointer) */
  JOLT_ENOSPACE = -2,   /* workspace or record buffer too small               */
  JOLT_EBUDGET = -3,    /* byte budget below the cheapest plan                */
  JOLT_ERANGE = -4,     /* non-finite input                                   */
  JOLT_EFORMAT = -5,    /* record header: bad magic, version or shape         */
  JOLT_EHIP = -6,       /* HIP runtime error (launch, copy or device fault)   */
  JOLT_ENODEV = -7      /* no usable gfx950 device                            */
} jolt_status;

typedef enum { JOLT_BF16 = 0, JOLT_F32 = 1 } jolt_dtype;
typedef enum { JOLT_EXACT = 0, JOLT_FLASH = 1 } jolt_method;

/* Shape of one K or V tensor of one layer. */
typedef struct {
  int32_t H, T, D;      /* heads, tokens, features (D == 128)                */
  int32_t dtype;        /* jolt_dtype of the input and of decoded output     */
} jolt_shape;

/* Ranks and residual bits of one tensor.  (0, 0, b) = no Tucker part: the
 * whole tensor is the residual.  Otherwise 1 <= r_T <= H*D, 1 <= r_D <= D
 * (a record may hold fewer tokens than r_T: see jolt_append).  bits in 1..4. */
typedef struct { int32_t r_T, r_D, bits; } jolt_choice;

/* Allocation request for a whole cache: n_layers layers x {K, V}, all of one
 * shape.  Tensor index i = layer * 2 + kind (kind 0 = K, 1 = V).
 * Source: JoLT abstract, the sentence on the single Lagrangian dual that
 * allocates Tucker ranks and residual bit-widths per layer group, keys and
 * values separately, under one byte budget. */
typedef struct {
  jolt_shape shape;
  int32_t n_layers;
  int32_t group_layers;   /* layers per allocation group (4)                  */
  double budget_ratio;    /* budget = floor(2 * H*T*D * 2*n_layers / ratio) B  */
  int32_t bit_menu[4];    /* residual bit-widths offered, each in 1..4         */
  int32_t n_bits;         /* 1..4                                              */
  int32_t method;         /* jolt_method                                       */
  int32_t oversample;     /* FlashJoLT sketch oversampling p (10)              */
  int32_t power_iters;    /* FlashJoLT power iterations q (1)                  */
  int32_t r_T_cap;        /* 0 = min(T, HD, floor(Bbar/(4T)) to a step multiple)*/
  int32_t step_T, step_D; /* rank grid steps (0 = 32 and 16)                   */
  uint64_t seed;          /* seeds the sketch (FlashJoLT) and the rotation     */
} jolt_alloc_req;

/* Allocation result.  Host arrays are caller-owned; optional ones may be NULL. */
typedef struct {
  jolt_choice* choice;       /* out [n_groups * 2], index g * 2 + kind         */
  uint64_t* tensor_bytes;    /* out, optional [2 * n_layers]                   */
  double* spectra_T;         /* out, optional [2 * n_layers][jolt_spectrum_len]*/
  double* spectra_D;         /* out, optional [2 * n_layers][D]                */
  double* frob2;             /* out, optional [2 * n_layers]: ||X||_F^2        */
  double objective;          /* out: predicted sum of relative squared errors  */
  uint64_t total_bytes;      /* out: bytes of all records under the plan       */
  uint64_t budget_bytes;     /* out                                            */
  int32_t r_T_cap;           /* out: columns of U_T kept per tensor            */
} jolt_plan;

/* ---------------------------------------------------------------- sizes */

/* Bytes of one compressed record: a 64-byte header padded to 256, then
 * 256-aligned sections U_T bf16 [T][r_T], U_D bf16 [D][r_D], core bf16
 * [H][r_T][r_D], scales bf16 [H][T][D/32][2] (offset, step), codes
 * [H][T][D/32][4*bits] bytes.  0 if the arguments are invalid. */
size_t jolt_blob_bytes(const jolt_shape* shape, jolt_choice choice);

/* Device workspace needed by jolt_allocate for the request (0 if invalid). */
size_t jolt_workspace_bytes(const jolt_alloc_req* req);

/* Length of each token-mode spectrum jolt_allocate reports: the cap r_T_cap
 * (the leading eigenvalues that the allocator and the factors use). */
int32_t jolt_spectrum_len(const jolt_alloc_req* req);

/* Device workspace of jolt_encode / jolt_decode for one tensor. */
size_t jolt_encode_workspace_bytes(const jolt_shape* shape, jolt_choice choice);
size_t jolt_decode_workspace_bytes(const jolt_shape* shape, jolt_choice choice);
size_t jolt_decode_many_workspace_bytes(int32_t n, const jolt_shape* shape,
                                        const jolt_choice* choices);
/* Device workspace of jolt_encode_many (0 if the arguments are invalid). */
size_t jolt_encode_many_workspace_bytes(int32_t n, const jolt_shape* shape,
                                        const jolt_choice* choices);

/* Bytes of a prepared rotation (jolt_rotation). */
size_t jolt_rotation_bytes(int32_t D);

/* ------------------------------------------------------------ hot path */

/* Spectra, factors and allocation for a whole cache.
 * x_dev[i] (i = layer * 2 + kind) points at tensor i on the device.
 * Computes, per tensor, ||X||^2, the token- and feature-mode spectra and
 * orthonormal fp32 factors (U_T: r_T_cap columns, U_D: D columns) by Gram
 * eigendecomposition (method EXACT) or the seeded randomized SVD (FLASH),
 * keeps the factors in ws_dev (read them with jolt_factors), copies the
 * spectra to the host (the only synchronization: it waits on `stream`), and
 * runs the Lagrangian dual (jolt_plan_from_spectra).  ws_bytes must be at
 * least jolt_workspace_bytes(req).  Errors: EINVAL, ENOSPACE, EBUDGET,
 * ERANGE (non-finite ||X||^2), EHIP. */
jolt_status jolt_allocate(const jolt_alloc_req* req, const void* const* x_dev,
                          void* ws_dev, size_t ws_bytes, void* stream,
                          jolt_plan* plan);

/* Device addresses of tensor i's factors inside a workspace filled by
 * jolt_allocate: U_T fp32 [T][ld_T] (ld_T = r_T_cap, leading columns first)
 * and U_D fp32 [D][D].  Pure pointer arithmetic, no device access. */
jolt_status jolt_factors(const jolt_alloc_req* req, void* ws_dev, int32_t tensor,
                         const float** U_T, int32_t* ld_T, const float** U_D);
/* jolt_factors of tensors first .. first + n - 1 in one call: U_T[i],
 * ld_T[i] and U_D[i] (arrays of n, caller-owned) describe tensor first + i.
 * Errors: EINVAL (invalid request, range outside the cache's 2 L tensors,
 * NULL arrays with n > 0). */
jolt_status jolt_factors_many(const jolt_alloc_req* req, void* ws_dev, int32_t first, int32_t n,
                              const float** U_T, int32_t* ld_T, const float** U_D);

/* The seeded rotation Q (D x D, Haar: QR of a counter-based Gaussian matrix
 * with diag(R) > 0), prepared on the host in fp64 and uploaded to q_dev
 * (jolt_rotation_bytes(D) bytes: fp32 Q, fp32 Q^T, bf16 Q^T and the three
 * bf16 parts hi, mid, lo of the fp32 Q (hi + mid + lo = Q exactly, in the
 * matrix-core fragment order of the encoder), each section 256-aligned).  Synchronizes `stream`.
 * Source: JoLT abstract, the method sentence (the residual is rotated by a
 * random orthogonal matrix before low-bit quantization); news article on
 * JoLT, paragraph 4 (the rotation whitens the residual). */
jolt_status jolt_rotation(uint64_t seed, int32_t D, void* q_dev, size_t q_bytes,
                          void* stream);

/* A prepared rotation from a caller's D x D orthogonal matrix Q (fp64,
 * row-major, host; |Q^T Q - I| <= 1e-12 entrywise, else EINVAL), in the
 * layout of jolt_rotation.  With Q = I the residual path quantizes the
 * unrotated residual: the unrotated quantization baseline.  Synchronizes
 * `stream`.  Source: as jolt_rotation; the baseline: JoLT abstract, the
 * sentence naming per-entry quantization among the compared families. */
jolt_status jolt_rotation_from(const double* Q, int32_t D, void* q_dev, size_t q_bytes, void* stream);

/* Encode one tensor with the given factors: stores bf16 U_T[:, :r_T],
 * U_D[:, :r_D] and core G_h = U_T^T X_h U_D, takes the residual against the
 * stored parts, rotates it (Y = R Q^T along features), quantizes Y in groups
 * of 32 with per-group bf16 (offset, step) and packs the codes.  U_T_dev is
 * fp32 [T][ld_T], U_D_dev fp32 [D][ld_D]; rot_dev is a prepared rotation.
 * blob_bytes >= jolt_blob_bytes, ws_bytes >= jolt_encode_workspace_bytes.
 * Every buffer is caller-owned and must stay valid until `stream` has run
 * the call's work; the record is written on the stream, the inputs only read.
 * Asynchronous.  Errors: EINVAL, ENOSPACE, EHIP.
 * Source: JoLT abstract, the method sentences (partial Tucker decomposition
 * of the token and feature axes only, the head axis left intact; the energy
 * the truncation drops restored by a randomly rotated low-bit residual);
 * news article on JoLT, paragraphs 2 and 4. */
jolt_status jolt_encode(const jolt_shape* shape, const void* x_dev, jolt_choice choice,
                        const float* U_T_dev, int32_t ld_T,
                        const float* U_D_dev, int32_t ld_D,
                        const void* rot_dev, uint64_t seed,
                        void* blob_dev, size_t blob_bytes,
                        void* ws_dev, size_t ws_bytes, void* stream);

/* Encode n tensors of one shape: record i from x_dev[i] with choices[i] and
 * the factors U_T_dev[i] (fp32 [T][ld_T[i]]) and U_D_dev[i] (fp32
 * [D][ld_D[i]]) into blob_dev[i] (blob_bytes[i] >= jolt_blob_bytes).  The
 * records are those jolt_encode writes, byte for byte (the same kernels and
 * arithmetic, batched over the tensors of each (r_T, r_D) and over all
 * tensors for the residual, rotation and quantization); the factor arrays
 * may be NULL when no choice has r_T > 0.  All arrays are host arrays of
 * length n; the device pointers must stay valid until the stream reaches the
 * end of the call's work.  ws_bytes >= jolt_encode_many_workspace_bytes.
 * Synchronizes `stream` once (uploading the pointer tables), then
 * asynchronous.  Errors: EINVAL, ENOSPACE, EHIP.
 * Source: JoLT abstract (the compressed cache: Tucker parts plus the
 * JL-rotated, quantized residual of every layer's K and V). */
jolt_status jolt_encode_many(int32_t n, const jolt_shape* shape, const jolt_choice* choices,
                             const void* const* x_dev, const float* const* U_T_dev,
                             const int32_t* ld_T, const float* const* U_D_dev,
                             const int32_t* ld_D, const void* rot_dev, uint64_t seed,
                             void* const* blob_dev, const size_t* blob_bytes,
                             void* ws_dev, size_t ws_bytes, void* stream);

/* Decode one record: X^_h = U_T G_h U_D^T + dequant(codes)_h Q, written to
 * xhat_dev in shape->dtype.
 * Source: JoLT abstract, the method sentences (the Tucker reconstruction plus
 * the rotated residual restores the cache; quality is the relative Frobenius
 * error of this reconstruction).
 * The decode trusts its caller: shape and choice must be those the record
 * was encoded with (jolt_header_parse reads them from a host copy of the
 * header); the device-side header is not read, so a mismatch is not detected
 * and gives wrong output inside the buffers the arguments describe.  ws_bytes
 * >= jolt_decode_workspace_bytes.  Asynchronous.
 * Arithmetic: bf16 matrix cores with fp32 accumulation; W = G_h U_D^T is
 * carried as a hi + lo bf16 pair, the dequantized residual and Q in bf16.
 * xhat_dev [H][T][D] row-major, caller-owned; it needs only the element's own
 * alignment (outputs on 16-byte boundaries are written 16 bytes at a time,
 * others one element at a time, with identical values). */
jolt_status jolt_decode(const jolt_shape* shape, jolt_choice choice,
                        const void* blob_dev, size_t blob_bytes,
                        const void* rot_dev, void* xhat_dev,
                        void* ws_dev, size_t ws_bytes, void* stream);

/* Decode n records of one shape in few launches (up to 32 records each):
 * record i (choices[i], blobs[i] of blob_bytes[i]) into outs[i].  Same
 * arithmetic as jolt_decode.  ws_bytes >= jolt_decode_many_workspace_bytes.
 * Source: JoLT abstract (reconstruction of the whole cache, whose error the
 * paper reports as relative Frobenius error). */
jolt_status jolt_decode_many(int32_t n, const jolt_shape* shape, const jolt_choice* choices,
                             const void* const* blobs, const size_t* blob_bytes,
                             const void* rot_dev, void* const* outs,
                             void* ws_dev, size_t ws_bytes, void* stream);

/* ---------------------------------------------------- appended tokens */

/* Incremental encode of n_new tokens appended to a tensor already encoded
 * (base_blob: shape `base`, choice with r_T > 0): the pages are silent on
 * tokens that arrive after encoding; the reading is folding-in (new rows fit
 * to fixed factors, as latent semantic indexing adds documents without a new
 * SVD).  The base's stored U~_D and G~ are kept; the new tokens' token-factor
 * rows solve min_U ||X_new,(T) - U W||_F, W = [G~_h U~_D^T]_h (r_T x H D),
 * through the normal equations W W^T = Z diag(lambda) Z^T (the tridiagonal
 * eigensolver, fp32; only non-positive eigenvalues are dropped); the residual against the stored
 * parts is rotated and quantized as in jolt_encode.  Output: a record of
 * shape (H, n_new, D) with the base's choice (jolt_blob_bytes of that shape),
 * holding copies of U~_D and G~, which decodes (and attends) like any
 * record.  x_new_dev [H][n_new][D] in base->dtype.  ws_bytes >=
 * jolt_append_workspace_bytes.  Synchronizes `stream` once, at the end.
 * Errors: EINVAL, ENOSPACE, EHIP. */
size_t jolt_append_workspace_bytes(const jolt_shape* base, jolt_choice choice, int32_t n_new);
jolt_status jolt_append(const jolt_shape* base, jolt_choice choice, const void* base_blob, size_t base_bytes,
                        const void* x_new_dev, int32_t n_new, const void* rot_dev, uint64_t seed,
                        void* blob_dev, size_t blob_bytes, void* ws_dev, size_t ws_bytes, void* stream);

/* ------------------------------------------ decode fused into attention */

/* Attention of new query vectors over one layer's compressed K and V
 * records, with the records decoded tile by tile in registers (the decode's
 * arithmetic) and never written to memory.  Source: JoLT abstract, first
 * sentence (the KV cache is the dominant serving cost; attention is what
 * reads it); the consumer is not on the pages: plain scaled dot-product
 * attention, grouped as in GQA.
 * shape: the records' (H KV heads, T tokens, D = 128, dtype); choice_k /
 * choice_v: the records' choices (trusted, as in jolt_decode); q_dev fp32
 * [H * G][n_new][D] (query head h G + g attends over KV head h), out_dev
 * fp32 of the same layout: out = softmax(q K^T / sqrt(D)) V.  G * n_new <= 8.
 * ws_bytes >= jolt_attend_workspace_bytes (the two records' W planes and
 * per-block softmax partials).  Asynchronous.  Errors: EINVAL, ENOSPACE,
 * EHIP. */
size_t jolt_attend_workspace_bytes(const jolt_shape* shape, jolt_choice choice_k, jolt_choice choice_v,
                                   int32_t G, int32_t n_new);
jolt_status jolt_attend(const jolt_shape* shape, jolt_choice choice_k, const void* blob_k, size_t blob_k_bytes,
                        jolt_choice choice_v, const void* blob_v, size_t blob_v_bytes, const void* rot_dev,
                        const float* q_dev, int32_t G, int32_t n_new, float* out_dev, void* ws_dev,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------- cross-layer SVD baseline */

/* A comparison codec the pages name but do not define (JoLT abstract, the
 * sentence on cross-layer low-rank factorizations among the compared
 * families; news article on JoLT, paragraph 3): one feature basis for n
 * tensors of one shape (a layer group's K or V tensors), the leading r
 * eigenvectors U of their summed feature Grams sum_i sum_h X_ih^T X_ih
 * (tridiagonal eigensolver, fp32), stored as bf16 basis_dev [r][D] (row j =
 * eigenvector j, eigenvalues descending); each tensor stores its
 * coefficients bf16(X_i U~) as coeff_dev[i] [H][T][r]; reconstruction
 * X^_i = C_i U~^T in the input dtype.  Bytes: 2 H T r per tensor + 2 D r.
 * lam_host (optional, [r]): the leading eigenvalues.  ws_bytes >=
 * jolt_xl_workspace_bytes.  Synchronizes `stream` once, at the end.
 * Errors: EINVAL, ENOSPACE, EHIP. */
size_t jolt_xl_workspace_bytes(int32_t n, const jolt_shape* shape, int32_t r);
jolt_status jolt_xl_encode(int32_t n, const jolt_shape* shape, const void* const* x_dev, int32_t r,
                           void* basis_dev, void* const* coeff_dev, double* lam_host,
                           void* ws_dev, size_t ws_bytes, void* stream);
/* X^_i = C_i U~^T into out_dev[i] ([H][T][D], shape->dtype).  Asynchronous. */
jolt_status jolt_xl_decode(int32_t n, const jolt_shape* shape, int32_t r, const void* basis_dev,
                           const void* const* coeff_dev, void* const* out_dev, void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): jolt_decode_many without a workspace argument.  Its scratch
 * (the W = G U_D^T planes of the records of one launch) is a file-scope
 * device array of jolt_decode_static_scratch_bytes() bytes (32 MiB), one
 * copy per GPU, held until the process ends; its address is looked up once
 * per device on the first call there.  The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.  Records are
 * decoded in launches whose planes fit the array (so more launches than
 * jolt_decode_many when they do not all fit), with the same kernels and
 * arithmetic: the output is identical.  Errors: EINVAL as jolt_decode_many;
 * ENOSPACE when a blob is short or one record's planes (2 * 256-aligned
 * 2 H D ceil32(r_T) bytes) exceed the array.  Every call on one GPU shares
 * that GPU's array, so calls that overlap in time on one GPU (other streams,
 * other threads) race on it and must be serialized by the caller.
 * Asynchronous. */
size_t jolt_decode_static_scratch_bytes(void);
jolt_status jolt_decode_many_static(int32_t n, const jolt_shape* shape, const jolt_choice* choices,
                                    const void* const* blobs, const size_t* blob_bytes,
                                    const void* rot_dev, void* const* outs, void* stream);

/* Group quantizer alone (rows == 0 is a no-op; pointers may then be NULL):
 * rows x D fp32 rotated residual in y_dev ->
 * scales bf16 [rows][D/32][2] and packed codes [rows][D/32][4*bits].
 * The same arithmetic as the encode kernel's last stage. */
jolt_status jolt_quantize(const float* y_dev, int64_t rows, int32_t D, int32_t bits,
                          void* scales_dev, void* codes_dev, void* stream);

/* ------------------------------------------------------ host-only helpers */

/* The Lagrangian dual alone, on host spectra (no device access).
 * spectra_T: [2*n_layers][len_T], spectra_D: [2*n_layers][D], frob2:
 * [2*n_layers]; plan->choice must be allocated. */
jolt_status jolt_plan_from_spectra(const jolt_alloc_req* req, const double* spectra_T,
                                   int32_t len_T, const double* spectra_D,
                                   const double* frob2, jolt_plan* plan);

/* The rotation Q in fp64 on the host (D*D values, row-major). */
jolt_status jolt_rotation_host(uint64_t seed, int32_t D, double* Q);

/* Normal number `index` of the counter-based stream (seed, tag), fp64. */
double jolt_rng_normal(uint64_t seed, uint64_t tag, uint64_t index);

/* Parse a 64-byte record header. */
jolt_status jolt_header_parse(const void* header, size_t bytes, jolt_shape* shape,
                              jolt_choice* choice, uint64_t* seed);

const char* jolt_status_str(jolt_status s);
int32_t jolt_version(void);

/* Testing hook, process-wide and not for concurrent use: the polls a bulge-
 * chase wave of the eigensolver makes while waiting for its predecessor
 * before it gives up (default 2^22, restored by a negative value).  A wait
 * that gives up makes jolt_allocate return JOLT_EHIP; every kernel still
 * ends normally.  Lets a test force that error path from the host. */
void jolt_debug_chase_wait_limit(int32_t polls);

/* ------------------------------------------------------------ profiling */

/* Per-kernel statistics of the calls made while profiling was on: launches,
 * summed HIP-event time of those launches on their streams, and the
 * algorithmic HBM bytes and flops of the work they performed, as each launch
 * accounts it on the host (operands read once, outputs written once; the
 * flops the method needs, not the ones a kernel spends on its own scheme). */
typedef struct {
  int64_t launches;
  double total_ms;
  double bytes;
  double flops;
} jolt_kernel_stats;

/* Select the kernels to profile: a comma-separated list of names, "*" for
 * all, NULL or "" to turn profiling off.  Every call synchronizes the device
 * and clears the records.  While on, the library records two HIP events
 * around each launch of a selected kernel on its stream (host objects, no
 * device memory).  Not safe with concurrent hot-path calls on other
 * streams.  Kernel names: "qr_panel", "qr_update" (block reflectors applied
 * to tall blocks), "cholqr" (CholeskyQR of the factors, with its products as
 * "cholqr_gemm"), "gemm" (fp32 matrix-core products), "gemm_bf16" (bf16
 * matrix-core products), "band", "chase", "tri_eig", "chase_back",
 * "band_back" (the eigensolver stages), "gram" (the Grams), "encode_w",
 * "encode_residual", "quantize", "decode_w", "decode", "attend". */
jolt_status jolt_profile_enable(const char* kernels);

/* Synchronizes the device, then reports the statistics of one kernel name
 * (zeros if it never ran). */
jolt_status jolt_profile_query(const char* kernel, jolt_kernel_stats* out);

#ifdef __cplusplus
}
#endif
#endif /* JOLT_H */
