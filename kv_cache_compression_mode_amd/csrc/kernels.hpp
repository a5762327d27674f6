// Host-side launch interface of the codec's HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jolt {

enum { kBF16 = 0, kF32 = 1 };

// ---- opt-in profiling (jolt_profile_enable): HIP events around launches of a
// selected kernel on its stream, and the algorithmic bytes and flops that the
// host code issuing the launch accounts for it.
bool prof_enabled(const char* name);
void prof_add_work(const char* name, double bytes, double flops);
struct ProfScope {
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  const char* name;
  hipStream_t stream;
  int e0, e1;   // event-pool slots, -1 when not recording
};

// offset(i) = (i / len) * seg + (i % len) * stride   (len = INT64_MAX: plain stride)
struct GemmDim {
  int64_t len, seg, stride;
};
inline GemmDim plain(int64_t stride) { return GemmDim{INT64_MAX, 0, stride}; }
inline GemmDim segmented(int64_t len, int64_t seg, int64_t stride) { return GemmDim{len, seg, stride}; }

// C[z](m, n) = alpha * sum_k A[z](m, k) B[z](k, n) * col_scale[z][n] + beta * C[z](m, n) (or c_in)
struct GemmArgs {
  int64_t M, N, K;
  const void* A; int a_dtype; GemmDim am, ak; int64_t a_batch;
  const void* B; int b_dtype; GemmDim bk, bn; int64_t b_batch;
  const void* const* a_ptrs;   // optional device array: operand base per batch entry
  const void* const* b_ptrs;
  void* C; int c_dtype; int64_t c_m, c_n, c_batch;
  void* const* c_ptrs;         // optional device array: output base per batch entry
  // optional fp32 source of the beta term, laid out as C (plain C only):
  // C = alpha A B + beta c_in, so that C need not hold a copy beforehand
  const float* c_in;
  float alpha, beta;
  const float* col_scale; int64_t col_scale_batch;
  // split-K: ksplit > 1 writes partial sums to `partial` ([batch][ksplit][M][N]
  // floats) and reduces them in a fixed order (deterministic)
  int ksplit; float* partial; int64_t kchunk;
  // split_seq (bf16 tiles): with ksplit > 1, the same K chunks are summed in
  // the same order inside one workgroup (no partial sums in memory), so the
  // result is bit-identical to the split launch; seq_len is set by the launcher
  int split_seq; int64_t seq_len;
  // symmetric operands stored as their lower triangle (fp32 path, plain
  // dimensions only): a_sym reads A(m, k) with m < k from A(k, m); c_lower
  // computes and writes only C(m, n) with m >= n (the launcher may pass -1,
  // m <= n, to a kernel computing the transposed product)
  int a_sym, c_lower;
  // the a_ptrs / b_ptrs entries are 16-byte aligned
  int ptr_align16;
  // both operands fp32 may run on bf16 matrix cores as hi + lo planes (1:
  // four products, about 2^-17 relative error per term instead of fp32's
  // 2^-24; 3: the same without lo x lo, 2^-16, for products whose result is a
  // small correction) or, both k contiguous, as three planes (2: six
  // products, about 2^-24)
  int split_f32;
  // triangular operands (matrix-core path): A(m, k) = 0 for k > m (a_lower),
  // B(k, n) = 0 for k > n (b_upper); a tile's K range then ends at its last
  // row (column)
  int a_lower, b_upper;
};

// scope: the profiling name of the launch (default "gemm_bf16" or "gemm" by the units it runs on)
hipError_t launch_gemm(const GemmArgs& g, int batch, hipStream_t s, const char* scope = nullptr);
hipError_t launch_sumsq(const void* const* xs_dev, int ntensors, int64_t n, int dtype, double* out,
                        hipStream_t s);
// Gaussian sketch per tensor, column-major [cols][rows] (element (i, j) is
// normal number i * cols + j of the tensor's stream).
hipError_t launch_sketch(float* out, int64_t rows, int64_t cols, uint64_t seed, const uint64_t* tags,
                         int ntensors, hipStream_t s);
hipError_t launch_to_bf16(const float* in, int64_t ld_in, uint16_t* out, int64_t rows, int64_t cols,
                          hipStream_t s);
hipError_t launch_to_bf16_many(const float* const* ins_dev, int64_t ld_in, uint16_t* const* outs_dev, int64_t rows,
                               int64_t cols, int n, hipStream_t s);
hipError_t launch_row_sumsq(const float* P, int64_t rows, int64_t cols, int64_t batch_stride,
                            int batch, double* out, int64_t out_batch, hipStream_t s);
hipError_t launch_col_dot(const float* A, const float* B, int64_t m, int64_t ncols, int64_t ld,
                          int64_t batch_stride, int batch, double* out, int64_t out_batch, hipStream_t s);
hipError_t launch_pad_copy(const float* in, int64_t n, int64_t in_batch, float* out, int64_t n_pad,
                           int batch, hipStream_t s);
hipError_t launch_sum_diag_blocks(const float* C, int64_t H, int64_t D, float* GD, int batch,
                                  hipStream_t s);
// The diagonal of M (np x np) past the leading n x n block set to the
// block's largest diagonal entry.
hipError_t launch_pad_diag(float* M, int64_t n, int64_t np, hipStream_t s);
// inv[i] = 1 / lam[i] for lam[i] > rel * max(lam), else 0 (lam fp64 [n]).
hipError_t launch_pinv_scale(const double* lam, int64_t n, double rel, float* inv, hipStream_t s);
// out[i] = sum_{j < n} in[j * count + i], added in the order j = 0 .. n-1.
hipError_t launch_sum_batch(const float* in, int64_t count, int n, float* out, hipStream_t s);

// ---- Householder QR, column-major panels [batch][k][ld] (column j at j*ld) ----
// In place: on return the panel holds the explicit orthonormal Q (m x k, m >= k)
// with diag(R) >= 0.  work: householder_qr_work_floats(m, k, batch) floats.
size_t householder_qr_work_floats(int64_t m, int64_t k, int batch);
// Householder factorization of the panel columns [c0, c0 + nb) (nb <= 32) of
// column-major m x k matrices (rows c0 .. m-1): explicit unit-lower V
// (m x 32, zero above row c0) -> Vp, compact-WY T (32 x 32 row-major) -> Tp,
// tau / sign(beta_j) -> taus[j] / taus[k + j] (per matrix 2k floats).  The
// panel's own columns in A are left as they were (the R factor is not
// written).  scratch: panel_factor_scratch_floats(m, batch) floats.
size_t panel_factor_scratch_floats(int64_t m, int batch);
// Top R eigenpairs of `batch` symmetric n x n matrices A (row-major = column-
// major; n a multiple of 32; A is destroyed) by two-stage tridiagonal
// reduction: Z [batch][n][n] receives the eigenvectors as the first R
// columns (column-major, ld n), eigenvalue-descending; lam (optional, fp64
// [batch][R]) the eigenvalues.  work: syev_top_work_bytes(n, R, batch).
size_t syev_top_work_bytes(int64_t n, int R, int batch);
// status: a device int the bulge chase ORs 1 into when one of its bounded
// waits gives up (cleared by the caller, read back at its next sync).
// band_done, when given, is recorded on s once the band reduction is queued.
// inv_sqrt_scale: eigenvector j comes out multiplied by 1 / sqrt(lam_j) where
// lam_j > 0 (so X v_j / sqrt(lam_j) has unit norm for the Gram of X).
// side, when given: a second stream of the caller and two events of its own,
// on which the chase back-transformation's block factors are formed beside
// the tridiagonal eigenpairs (they need the chase's reflectors only).
struct SyevSide {
  hipStream_t s;
  hipEvent_t chase_done, tfac_done;
};
hipError_t syev_top(float* A, int64_t n, int batch, int R, float* Z, double* lam, void* work, hipStream_t s,
                    int* status, hipEvent_t band_done = nullptr, bool inv_sqrt_scale = false,
                    const SyevSide* side = nullptr);
// Polls a bulge-chase wave makes before its wait gives up (default 2^22).
void set_chase_spin_limit(int polls);
hipError_t copy_cols(const float* in, int64_t ld_in, int64_t in_batch, float* out, int64_t ld_out,
                     int64_t out_batch, int64_t rows, int64_t cols, int batch, hipStream_t s);
// write_r: when the panel fits one block (m - c0 <= panel_block_rows()), R
// (upper triangle) is also written into the panel's top nb rows.
int64_t panel_block_rows();
hipError_t panel_factor(float* A, int64_t m, int64_t ld, int64_t bstride, int64_t c0, int nb, int batch,
                        float* Vp, int64_t vstride, float* Tp, int64_t tstride, float* taus, int64_t k,
                        float* scratch, hipStream_t s, int write_r = 0);
hipError_t householder_qr(float* A, int64_t m, int64_t k, int64_t ld, int64_t batch_stride, int batch,
                          float* work, hipStream_t s);

// Thin QR of a full-rank, nearly orthonormal tall column-major U (m x k,
// k <= cholesky_qr_max_k(); unit-norm columns up to a few percent) by one
// CholeskyQR pass: Q (U's shape: ld, bstride) receives the factor with
// Q^T Q = I and U = Q R, diag(R) > 0; U is read only.  work:
// cholesky_qr_work_floats(m, k, batch) floats.  A column far from orthogonal
// to the earlier ones (a pivot below half its original diagonal) ORs 2 into
// *status, and Q then holds no valid factor: the caller repeats with
// householder_qr.
int64_t cholesky_qr_max_k();
size_t cholesky_qr_work_floats(int64_t m, int64_t k, int batch);
hipError_t cholesky_qr(const float* U, float* Q, int64_t m, int64_t k, int64_t ld, int64_t bstride, int batch,
                       float* work, int* status, hipStream_t s);

// Sort columns by lam descending (ties: lower index), sign-fix (largest |.| entry
// positive, lowest index on ties) and emit row-major U_out [m][ld_out]; lam_out
// sorted, fp64.  perm / sign: [batch][R] scratch.
hipError_t finalize_factor_ws(const float* U_cm, int64_t m, int64_t R, int64_t ld_cm, int64_t cm_batch,
                              const double* lam, int64_t lam_batch, float* U_out, int64_t ld_out,
                              int64_t out_batch, double* lam_out, int64_t lam_out_batch, int batch,
                              int* perm, float* sign, hipStream_t s);

// ---- codec ----
hipError_t launch_quantize(const float* Y, int64_t rows, int bits, uint16_t* scales, uint8_t* codes,
                           hipStream_t s);
// W_h = G~_h U~_D^T (D = 128) as two bf16 parts (hi, lo) in matrix-core
// fragment order, W2[p][h][d / 32][k / 16][32 ((k / 8) % 2) + d % 32][k % 8]
// (p < 2, k < r_Tp, zero for k >= r_T; r_Tp a multiple of 64), of n tensors:
// tensor j reads G~_h from Gp[j H + h] and U~_D from Udp[j H + h] (G0 + h r_T
// r_D and Ud0 when Gp is null) and writes W2 + j w2_batch (2 H 128 r_Tp values
// per tensor).
hipError_t launch_enc_w(const uint16_t* const* Gp, const uint16_t* const* Udp, const uint16_t* G0,
                        const uint16_t* Ud0, uint16_t* W2, int64_t w2_batch, int n, int H, int r_T, int r_D,
                        int r_Tp, hipStream_t s);
// Fused residual -> rotation -> quantization for one tensor (D = 128).
struct EncodeArgs {
  const void* X; int x_dtype; int64_t H, T;
  const uint16_t* Ut;  // bf16 [T][r_T] (NULL when r_T == 0)
  const uint16_t* W2;  // the two bf16 parts of W_h in fragment order (launch_enc_w)
  int64_t r_T, r_Tp;
  const uint16_t* Q3;  // bf16 parts of Q in fragment order, [3][c / 32][d / 16][32 ((d / 8) % 2) + c % 32][d % 8]
                       // (the exact three-part split; the encoder reads parts 0 and 1)
  int bits;
  uint16_t* scales;    // [H][T][4][2]
  uint8_t* codes;      // [H][T][4][4*bits]
};
hipError_t launch_encode_residual(const EncodeArgs& a, hipStream_t s);
// n tensors of one shape (H, T), arguments in a device array
hipError_t launch_encode_residual_many(const EncodeArgs* list_dev, int n, int64_t H, int64_t T, int x_dtype,
                                       hipStream_t s);
// Batched decode: up to kDecBatch records of one shape (H, T, D = 128), all
// in one launch (the batch travels as the kernel argument, under its 4 KB
// limit).  A record is addressed by its base: its sections follow the record
// layout (bf16 U~_T [T][r_T] at byte 256, then U~_D [D][r_D], the core
// [H][r_T][r_D], the scale words [H][T][4] and the code words [H][T][4][bits],
// each section starting 256-aligned), which the host checks against the
// library's layout when it fills the record.
constexpr int kDecBatch = 64;
struct DecRec {
  const char* blob;
  void* out;               // [H][T][D]
  uint16_t* Whi;           // workspace: bf16 [H][D/32][r_Tp/16][64][8], fragment order; the lo plane follows
  int32_t H, T;
  int32_t r_T, r_D, r_Tp, bits;
  int32_t wtile0;          // first W tile of this record
  __host__ __device__ static size_t up256(size_t v) { return (v + 255) / 256 * 256; }
  __host__ __device__ size_t off_ud() const { return 256 + up256(2ull * T * r_T); }
  __host__ __device__ size_t off_g() const { return off_ud() + up256(2ull * 128 * r_D); }
  __host__ __device__ size_t off_sc() const { return off_g() + up256(2ull * H * r_T * r_D); }
  __host__ __device__ size_t off_cd() const { return off_sc() + up256(4ull * (static_cast<size_t>(H) * T * 128 / 32)); }
  __host__ __device__ const uint16_t* Ut() const { return reinterpret_cast<const uint16_t*>(blob + 256); }
  __host__ __device__ const uint16_t* Ud() const { return reinterpret_cast<const uint16_t*>(blob + off_ud()); }
  __host__ __device__ const uint16_t* G() const { return reinterpret_cast<const uint16_t*>(blob + off_g()); }
  __host__ __device__ const uint32_t* scales() const { return reinterpret_cast<const uint32_t*>(blob + off_sc()); }
  __host__ __device__ const uint32_t* codes() const { return reinterpret_cast<const uint32_t*>(blob + off_cd()); }
  __host__ __device__ uint16_t* Wlo() const { return Whi + up256(2ull * H * 128 * r_Tp) / 2; }
};
struct DecBatch {
  DecRec rec[kDecBatch];
  int32_t n, H, T, out_dtype, wtiles_total;
  int32_t out16;            // every record's out is 16-byte aligned
  const uint16_t* Qt16;    // bf16 [D][D], Qt16[c][d] = Q[d][c]
};
static_assert(sizeof(DecBatch) <= 4000, "a decode batch is one kernel argument");
hipError_t launch_decode_batch(const DecBatch& b, hipStream_t s);
// The W planes of the batch's records alone (the decode's prologue).
hipError_t launch_make_w(const DecBatch& b, hipStream_t s);

// Decode fused into attention over one layer's K and V records: per KV head
// h, nq = G * n_new query vectors (the GQA group's query heads times the new
// tokens), q fp32 [H * G][n_new][D] (query head h G + g reads KV head h),
// out fp32 of the same layout; part: fp32 [H][nq][n_blk][D + 2] block partials
// (o[D], max, sum), n_blk = ceil(T / 256).  The records' W planes must be
// formed beforehand (launch_make_w).
constexpr int kAttnMaxQ = 8;
struct AttnArgs {
  DecRec k, v;
  const uint16_t* Qt16;    // bf16 [D][D], Qt16[c][d] = Q[d][c]
  const float* q;
  float* out;
  float* part;
  float scale;             // 1 / sqrt(D)
  int32_t H, T, G, n_new, nq, n_blk;
};
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s);
// The 256-byte head of a record (the 64-byte header, zeros to 256) and the
// padding after each of its five sections, zeroed, so that every byte of a
// record is defined: pad[2 j] = byte offset, pad[2 j + 1] = length (< 256).
struct RecordHead {
  uint32_t w[16];
  uint32_t pad[10];
  uint32_t unused[6];
};
hipError_t launch_write_header(void* blob, const RecordHead& head, hipStream_t s);
// heads_dev[i] into blobs_dev[i], i < n
hipError_t launch_write_headers(uint32_t* const* blobs_dev, const RecordHead* heads_dev, int n, hipStream_t s);

}  // namespace jolt
