// Host-side launch interface of the codec's HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jolt {

enum { kBF16 = 0, kF32 = 1 };

// ---- opt-in profiling (jolt_profile_enable): HIP events around launches of a
// selected kernel on its stream, plus device counters (bytes, flops) that a
// kernel fills with the work it actually performed: one [2] slot per
// workgroup, each added to only by the workgroup of that grid position, so
// launches serialized on one stream accumulate without atomics.
bool prof_enabled(const char* name);
unsigned long long* prof_slots(const char* name, int64_t count);   // nullptr when off
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

// C[z](m, n) = alpha * sum_k A[z](m, k) B[z](k, n) * col_scale[z][n] + beta * C[z](m, n)
struct GemmArgs {
  int64_t M, N, K;
  const void* A; int a_dtype; GemmDim am, ak; int64_t a_batch;
  const void* B; int b_dtype; GemmDim bk, bn; int64_t b_batch;
  const void* const* a_ptrs;   // optional device array: operand base per batch entry
  const void* const* b_ptrs;
  void* C; int c_dtype; int64_t c_m, c_n, c_batch;
  void* const* c_ptrs;         // optional device array: output base per batch entry
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
};

hipError_t launch_gemm(const GemmArgs& g, int batch, hipStream_t s);
hipError_t launch_sumsq(const void* const* xs_dev, int ntensors, int64_t n, int dtype, double* out,
                        hipStream_t s);
hipError_t launch_sketch(float* out, int64_t rows, int64_t cols, uint64_t seed, const uint64_t* tags,
                         int ntensors, hipStream_t s);
hipError_t launch_to_bf16(const float* in, int64_t ld_in, uint16_t* out, int64_t rows, int64_t cols,
                          hipStream_t s);
hipError_t launch_to_bf16_many(const float* const* ins_dev, int64_t ld_in, uint16_t* const* outs_dev, int64_t rows,
                               int64_t cols, int n, hipStream_t s);
hipError_t launch_gather_cols(const float* in, int64_t ld_in, int64_t in_batch, const int* idx,
                              int64_t idx_batch, float* out, int64_t ld_out, int64_t out_batch,
                              int64_t rows, int64_t ncols, int batch, hipStream_t s);
hipError_t launch_row_sumsq(const float* P, int64_t rows, int64_t cols, int64_t batch_stride,
                            int batch, double* out, int64_t out_batch, hipStream_t s);
hipError_t launch_col_dot(const float* A, const float* B, int64_t m, int64_t ncols, int64_t ld,
                          int64_t batch_stride, int batch, double* out, int64_t out_batch, hipStream_t s);
hipError_t launch_pad_copy(const float* in, int64_t n, int64_t in_batch, float* out, int64_t n_pad,
                           int batch, hipStream_t s);
hipError_t launch_sum_diag_blocks(const float* C, int64_t H, int64_t D, float* GD, int batch,
                                  hipStream_t s);

// ---- symmetric eigensolver (block Jacobi) ----
// A: [batch][n][n] (n multiple of 64), V: [batch][n][n] (initialized by the solver).
struct JacobiWork {
  float* A; float* V; int64_t n; int batch;
  float* J;          // [batch][n/64][64][64]
  int* active;       // [batch][n/64]
  int* rot_count;    // [batch]
  float* tau_abs;    // [batch]
};
hipError_t jacobi_init(const JacobiWork& w, float tau_abs_rel, hipStream_t s);
hipError_t jacobi_round(const JacobiWork& w, int round, float tau_rel, hipStream_t s);
// Per matrix, kOffBlocks partial sums (off-diagonal squares, diagonal squares)
// in fp64: part[z][block][2].  The host adds them in a fixed order.
constexpr int kOffBlocks = 64;
hipError_t jacobi_offnorm(const float* A, int64_t n, int batch, double* part, hipStream_t s);
// Scalar Jacobi to convergence on 128 x 128 matrices (one workgroup each):
// A -> diagonal (in place), V <- eigenvectors.
hipError_t jacobi_small128(float* A, float* V, int batch, float tau_rel, float tau_abs_rel,
                           int max_sweeps, hipStream_t s);
// Indices of the R largest diagonal entries of each A, descending (ties: lower index).
hipError_t topk_diag(const float* A, int64_t n, int batch, int R, int* idx, hipStream_t s);

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
// band_done, when given, is recorded on s once the band reduction is queued
hipError_t syev_top(float* A, int64_t n, int batch, int R, float* Z, double* lam, void* work, hipStream_t s,
                    hipEvent_t band_done = nullptr);
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
// W_h = G~_h U~_D^T (D = 128) as three bf16 parts in matrix-core fragment
// order, W3[p][h][d / 32][k / 16][32 ((k / 8) % 2) + d % 32][k % 8] (k < r_Tp,
// zero for k >= r_T; r_Tp a multiple of 64), of n tensors: tensor j reads G~_h from Gp[j H + h] and
// U~_D from Udp[j H + h] (G0 + h r_T r_D and Ud0 when Gp is null) and writes
// W3 + j w3_batch.  r_Tp is a multiple of 32.
hipError_t launch_enc_w(const uint16_t* const* Gp, const uint16_t* const* Udp, const uint16_t* G0,
                        const uint16_t* Ud0, uint16_t* W3, int64_t w3_batch, int n, int H, int r_T, int r_D,
                        int r_Tp, hipStream_t s);
// Fused residual -> rotation -> quantization for one tensor (D = 128).
struct EncodeArgs {
  const void* X; int x_dtype; int64_t H, T;
  const uint16_t* Ut;  // bf16 [T][r_T] (NULL when r_T == 0)
  const uint16_t* W3;  // bf16 parts of W_h in fragment order (launch_enc_w)
  int64_t r_T, r_Tp;
  const uint16_t* Q3;  // bf16 parts of Q in fragment order, [3][c / 32][d / 16][32 ((d / 8) % 2) + c % 32][d % 8]
  int bits;
  uint16_t* scales;    // [H][T][4][2]
  uint8_t* codes;      // [H][T][4][4*bits]
};
hipError_t launch_encode_residual(const EncodeArgs& a, hipStream_t s);
// n tensors of one shape (H, T), arguments in a device array
hipError_t launch_encode_residual_many(const EncodeArgs* list_dev, int n, int64_t H, int64_t T, int x_dtype,
                                       hipStream_t s);
// Batched decode: up to kDecBatch records of one shape (H, T, D = 128).
constexpr int kDecBatch = 32;
struct DecRec {
  const uint16_t* Ut;      // bf16 [T][r_T]
  const uint16_t* Ud;      // bf16 [D][r_D]
  const uint16_t* G;       // bf16 [H][r_T][r_D]
  const uint32_t* scales;  // [H][T][4] words (offset | step << 16)
  const uint32_t* codes;   // [H][T][4][bits] words
  uint16_t* Whi;           // workspace: bf16 [H][D/32][r_Tp/16][64][8], fragment order
  uint16_t* Wlo;
  void* out;               // [H][T][D]
  int32_t r_T, r_D, r_Tp, bits;
  int32_t wtile0;          // first W tile of this record
};
struct DecBatch {
  DecRec rec[kDecBatch];
  int32_t n, H, T, out_dtype, wtiles_total;
  int32_t out16;            // every record's out is 16-byte aligned
  const uint16_t* Qt16;    // bf16 [D][D], Qt16[c][d] = Q[d][c]
};
hipError_t launch_decode_batch(const DecBatch& b, hipStream_t s);
hipError_t launch_write_header(void* blob, const uint32_t* words16, hipStream_t s);
// 16 words words_dev[i * 16 ..] into the header of blobs_dev[i], i < n
hipError_t launch_write_headers(uint32_t* const* blobs_dev, const uint32_t* words_dev, int n, hipStream_t s);

}  // namespace jolt
