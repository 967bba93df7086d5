// Internal interface between the host runtime (muon_api.cpp) and the HIP
// kernels (muon_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include "muon.h"

namespace muon {

// Matrices handled by one launch when the launch needs per-matrix pointers.
constexpr int kChunk = 64;
// Every workspace matrix is padded with zeros to a multiple of kPad in both
// dimensions, so the GEMM kernels never test bounds.
constexpr int kPad = 256;
// Tile of the elementwise prep kernel (oriented coordinates).
constexpr int kPrepTile = 64;

// GEMM epilogues: GRAM A = inv^2 X X^T; POLY B = b A + c A A; UPDATE
// X <- scl (a X + B X) written as the next X state; FINAL_W the same value
// subtracted (times lr * scale) from the weights; FINAL_OUT the same value
// written to the caller's output.  The _T variants are the FINALs of tall
// matrices (stored transposed to the oriented X).
enum Epi {
  EPI_GRAM = 0, EPI_POLY = 1, EPI_UPDATE = 2, EPI_FINAL_W = 3, EPI_FINAL_OUT = 4,
  EPI_FINAL_W_T = 5, EPI_FINAL_OUT_T = 6,
  EPI_GRAM_LO = 7,  // bf16 GRAM that also writes C's residual to Clo
  EPI_POLY_LO = 8,  // bf16 POLY whose A input is Ain + Alo
  EPI_UPDATE_ROWS = 9,  // bf16 UPDATE that also writes row sums of the new X^2
  EPI_FINAL_W_MIX = 10  // bf16 FINAL_W over wide and tall matrices in one launch,
                        // each matrix's orientation from tall_mask
};
enum Final { FINAL_NONE = 0, FINAL_OUT = 1, FINAL_WEIGHTS = 2 };

// Inputs of the prep kernel: momentum (step) or plain input (orthogonalize),
// Frobenius partial sums, and the oriented, zero-padded X_0 copies.
// X state between Newton-Schulz steps, oriented M x N per matrix:
//   bf16 compute: X = hi + lo, a bf16 plane hi and a plane lo of one signed
//                 byte per element, x - hi in 1/256 of hi's bf16 spacing
//                 (lo8_of, 16 significant bits in all); hi is also the MFMA
//                 operand and is double-buffered, because the update reads all
//                 of hi as its second operand while writing the next hi;
//   fp32 compute: X in fp32, plus X^T (N x M) as the update's operand.
struct PrepArgs {
  int m, n, M, N;          // oriented shape and its padded size
  unsigned long long tall_mask;  // bit i: matrix i is tall (rows = n, cols = m),
                                 // its oriented X is the original transposed
  int tiles_n;             // N / kPrepTile
  const void* in;          // orthogonalize: input base (matrix i at in + i*s_in)
  long long s_in;
  float mu;
  long long sX;            // per-matrix stride of the M x N planes
  void* Xh; void* Xl;      // bf16: hi, lo (bytes) of X_0
  float* Xf;               // fp32: X_0
  void* XT; long long sXT; // fp32: X_0^T, N x M
  float* partials;         // [matrix][tile] sum of u^2
  int nblk;                // tiles per matrix
  int stream;              // nontemporal accesses (the group's X state is large)
};

struct PrepTable {         // step only: per-matrix gradient / momentum pointers
  const void* g[kChunk];
  float* buf[kChunk];
};

// C[i][j] = sum_k P[i][k] Q[j][k] over a padded batch, with an epilogue.
// The bf16 UPDATE / FINAL take Q row-major instead (Q[k][j] at
// Q + k * ldq + j): their second operand is the hi plane of X itself.
struct GemmArgs {
  const void* P; const void* Q;
  long long sP, sQ;        // per-matrix strides, elements
  int ldp, ldq, K;
  int tiles_m, tiles_n;
  int tiles_per_mat;       // set by launch_gemm
  int mat0;                // the launch covers matrices mat0 .. mat0 + batch - 1
  int group_m;             // full grids: tile rows per scheduling group
  int tri;                 // 1: lower-triangle tiles only (GRAM, POLY)
  const float* inv;        // first step: 1/(||u||_F+eps) per matrix, else null
  float a, b, c;           // step coefficients
  // GRAM / POLY output (M x M), POLY input A
  void* C; long long sC; int ldc;
  const void* Ain; long long sAin;
  void* Clo;               // GRAM_LO: C's residual v - bf16(v), lower tiles only
  const void* Alo;         // POLY_LO: a residual plane added to Ain (same layout)
  // UPDATE / FINAL: X state (see PrepArgs), leading dimension ldx, stride sX
  long long sX; int ldx;
  const void* Xh; void* Xh_next; void* Xl;  // bf16: hi (read), next hi, lo (in place)
  float* Xf;                                 // fp32: X (in place)
  void* XTo; long long sXT; int ldxt;        // fp32: next step's X^T
  int m, n;
  unsigned long long tall_mask;          // bit i: matrix i is stored tall
  int final_mode;
  void* out; long long s_out; int out_bf16;
  int vec_tall;            // FINAL of tall matrices: 4 consecutive i of a
                           // weight / output row are 16- (8-) byte aligned
  int vec_wide;            // FINAL of wide matrices (bf16): 8 consecutive j
                           // of a weight / output row are 16-byte aligned
  float neg_lrwd;          // FINAL_W: -lr * weight_decay (0: no decay)
  int cautious;            // FINAL_W: decay only where O * W >= 0
  float neg_lr;
  int stream;              // UPDATE / FINAL: nontemporal X-state and weight accesses
  // UPDATE_ROWS: sum over each 64-column block jb of X'[i][j]^2 at
  // rowpart[mat * s_rp + jb * ld_rp + i]
  float* rowpart; long long s_rp; int ld_rp;
};

struct WeightTable {       // FINAL_WEIGHTS only
  float* w[kChunk];
  float scale[kChunk];
};

// The single kernel argument of each kernel (its tables are read in place
// from the kernarg segment).
struct PrepLaunch {
  PrepArgs a;
  PrepTable t;
};
struct GemmLaunch {
  GemmArgs a;
  WeightTable wt;
};

// NorMuon: per oriented row i of the final X (= O, m x n), in fixed order,
// s = sum_j O[i][j]^2, v[i] <- beta2 v[i] + (1 - beta2) s / n and
// rinv[i] = 1 / (sqrt(v[i]) + eps2) (0 for padding rows).
struct RowTable {          // per-matrix second-moment vectors, m floats each
  float* v[kChunk];
};
struct NormuonArgs {
  int m, n, M, N;
  long long sX; int ldx;   // X state as in GemmArgs
  const void* Xh; const void* Xl;  // bf16: hi, lo
  const float* Xf;                 // fp32: X
  // bf16: the last UPDATE's row sums (GemmArgs::rowpart), N / 64 per row,
  // summed here instead of reading X
  const float* rowpart; long long s_rp; int ld_rp;
  float beta2, eps2;
  float* rinv;             // [matrix][M]
};
struct NormuonLaunch {
  NormuonArgs a;
  RowTable t;
};

// The weight update as its own pass (after NorMuon): per element of W in
// the caller's orientation, with O from the oriented X state,
//   W <- W - lr*scale*O*rinv[i] - lr*wd*mask*W,  mask = (O*W >= 0) if cautious.
struct ApplyArgs {
  int m, n, M, N;
  unsigned long long tall_mask;
  int tiles_n;             // N / kPrepTile
  long long sX; int ldx;
  const void* Xh; const void* Xl; const float* Xf;
  const float* rinv;       // [matrix][M]
  float neg_lr;            // -lr
  float neg_lrwd;          // -lr * weight_decay
  int cautious;
};
struct ApplyLaunch {
  ApplyArgs a;
  WeightTable wt;
};

// Launchers (return hipGetLastError() of the launch).
hipError_t launch_prep(int grad_bf16, int compute_bf16, int momentum,
                       const PrepArgs& a, const PrepTable& t, int batch,
                       hipStream_t s);
hipError_t launch_norm(const float* partials, int nblk, float eps, float* inv,
                       int batch, hipStream_t s);
// Square GEMM tile edge (128 or 256) used for a compute precision, given
// the caller's preference (0 = default).
int gemm_tile(int compute_bf16, int tile_pref);
hipError_t launch_gemm(int compute_bf16, int epi, int tile, const GemmArgs& a,
                       const WeightTable& t, int batch, hipStream_t s);
hipError_t launch_normuon_rows(int compute_bf16, const NormuonArgs& a, const RowTable& t,
                               int batch, hipStream_t s);
hipError_t launch_apply(int compute_bf16, const ApplyArgs& a, const WeightTable& t,
                        int batch, hipStream_t s);

// Measurement probes (muon_peaks.hip).
hipError_t launch_mfma_probe(int blocks, int iters, float* sink, hipStream_t s);
hipError_t launch_copy_probe(const void* src, void* dst, long long n16, int blocks,
                             hipStream_t s);

// Where a step's workspace comes from when the caller passes none
// (muon_step_static): asked once every argument has passed its checks, for
// `need` bytes; returns a muon_status.
struct WorkspaceSource {
  int (*get_fn)(const void* ctx, size_t need, void** ws, size_t* bytes);
  const void* ctx;
  int get(size_t need, void** ws, size_t* bytes) const { return get_fn(ctx, need, ws, bytes); }
};

// muon_step with its workspace from `src` (muon_api.cpp).
int step_with_source(int n, const int* rows, const int* cols, void* const* params,
                     int param_dtype, const void* const* grads, int grad_dtype,
                     float* const* momentum, float mu, float lr, const float* scale,
                     const muon_coeff* coeffs, int n_steps, float eps, int compute,
                     const WorkspaceSource& src, hipStream_t stream);

}  // namespace muon
