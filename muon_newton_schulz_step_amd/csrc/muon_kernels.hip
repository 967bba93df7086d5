// HIP kernels of the Muon step for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// Page 1 (web3.cnoyu.systems review of karpathy/autoresearch's train.py,
// Muon paragraph) defines the step: Nesterov momentum, Newton-Schulz
// iterations on A = X X^T with X <- aX + (bA + cA^2)X (tall matrices use the
// transposed form), then the orthogonal factor updates the weights.
//
// Kernels (one launch each per oriented shape group and step):
//   prep_kernel    momentum + Frobenius partial sums + oriented, zero-padded X_0
//   norm_kernel    fixed-order reduction of the partials -> 1/(||u||_F + eps)
//   gemm_kernel    C[i][j] = sum_k P[i][k] Q[j][k] on MFMA, three epilogues:
//                    GRAM   A = X X^T        (lower-triangle tiles, mirrored)
//                    POLY   B = b A + c A A  (A symmetric, so A A = A A^T)
//                    UPDATE X <- a X + B X   (Q = X^T, kept as its own copy)
// The 1/||u|| normalisation is folded into the first GRAM (x inv^2) and
// UPDATE (x inv) epilogues; the last UPDATE writes the weights (or the
// output) in the caller's orientation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_kernels.h"

namespace muon {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return static_cast<bf16_t>(x);  // v_cvt_pk_bf16_f32: round to nearest even
}

// ---------------------------------------------------------------- prep
// One 64x64 tile of the oriented, padded M x N space per block.  Reads the
// original matrix coalesced along its rows, writes the copy that shares the
// original layout directly and the transposed copy through an LDS tile.
template <typename GT, typename CT, bool MOM>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a, PrepTable t) {
  __shared__ float tile[kPrepTile][kPrepTile + 1];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int mat = blockIdx.y;
  const int bt = blockIdx.x;
  const int oi0 = (bt / a.tiles_n) * kPrepTile;
  const int oj0 = (bt % a.tiles_n) * kPrepTile;
  const bool tall = (a.tall_mask >> mat) & 1ull;
  const int rows = tall ? a.n : a.m, cols = tall ? a.m : a.n;  // original shape
  const int r0 = tall ? oj0 : oi0;  // tile origin in original coordinates
  const int c0 = tall ? oi0 : oj0;

  const GT* g;
  float* buf = nullptr;
  if constexpr (MOM) {
    g = static_cast<const GT*>(t.g[mat]);
    buf = t.buf[mat];
  } else {
    g = static_cast<const GT*>(a.in) + (long long)mat * a.s_in;
  }
  float* Xf = a.Xf + (long long)mat * a.sXf;
  bf16_t* Xb = a.Xb ? static_cast<bf16_t*>(a.Xb) + (long long)mat * a.sXf : nullptr;
  CT* XT = static_cast<CT*>(a.XT) + (long long)mat * a.sXT;

  const int cc = tid & 63, rr = tid >> 6;
  float sum = 0.f;
#pragma unroll 4
  for (int p = 0; p < kPrepTile / 4; ++p) {
    const int lr = rr + 4 * p;
    const int r = r0 + lr, c = c0 + cc;
    float u = 0.f;
    if (r < rows && c < cols) {
      const long long idx = (long long)r * cols + c;
      const float gv = to_f32(g[idx]);
      if constexpr (MOM) {
        const float nb = a.mu * buf[idx] + gv;  // buf' = mu*buf + g
        buf[idx] = nb;
        u = gv + a.mu * nb;                     // u = g + mu*buf'
      } else {
        u = gv;
      }
    }
    sum += u * u;
    if (!tall) {  // X[oi][oj] = X[r][c]
      const long long o = (long long)r * a.N + c;
      Xf[o] = u;
      if (Xb) Xb[o] = from_f32<bf16_t>(u);
    } else {        // X^T[oj][oi] = X^T[r][c]
      XT[(long long)r * a.M + c] = from_f32<CT>(u);
    }
    tile[lr][cc] = u;
  }
  __syncthreads();
#pragma unroll 4
  for (int p = 0; p < kPrepTile / 4; ++p) {
    const int lc = rr + 4 * p;
    const float u = tile[cc][lc];
    const int r = r0 + cc, c = c0 + lc;
    if (!tall) {  // X^T[oj][oi] = X^T[c][r]
      XT[(long long)c * a.M + r] = from_f32<CT>(u);
    } else {        // X[oi][oj] = X[c][r]
      const long long o = (long long)c * a.N + r;
      Xf[o] = u;
      if (Xb) Xb[o] = from_f32<bf16_t>(u);
    }
  }
  // Deterministic block sum: wave butterfly, then the four waves in order.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) a.partials[(long long)mat * a.nblk + bt] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------- norm
__global__ __launch_bounds__(256) void norm_kernel(const float* partials, int nblk,
                                                   float eps, float* inv) {
  __shared__ double red[256];
  const int mat = blockIdx.x, tid = threadIdx.x;
  double s = 0.0;
  for (int k = tid; k < nblk; k += 256) s += partials[(long long)mat * nblk + k];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) inv[mat] = (float)(1.0 / (sqrt(red[0]) + (double)eps));
}

// ---------------------------------------------------------------- GEMM
__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

template <typename T>
__device__ __forceinline__ void mma(f32x16_t& acc, const u32x4_t& fa, const u32x4_t& fb);

template <>
__device__ __forceinline__ void mma<bf16_t>(f32x16_t& acc, const u32x4_t& fa, const u32x4_t& fb) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa),
                                                __builtin_bit_cast(bf16x8_t, fb), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<float>(f32x16_t& acc, const u32x4_t& fa, const u32x4_t& fb) {
  // Four rank-2 steps; lane half h supplies k = 4h + e of this 8-wide chunk
  // pair, the same k for both operands, so the sum covers all 8 k once.
  const f32x4_t av = __builtin_bit_cast(f32x4_t, fa);
  const f32x4_t bv = __builtin_bit_cast(f32x4_t, fb);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], acc, 0, 0, 0);
}

// 128x128 output tile per block of 4 waves (2x2, 64x64 each, 2x2 MFMA 32x32
// tiles per wave).  K advances in steps of 128 bytes per row (64 bf16 or 32
// fp32), staged through two LDS buffers; 16-byte chunks of a row are stored
// at chunk ^ (row & 7) so that the MFMA operand reads are conflict-free.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a, WeightTable wt) {
  constexpr int BM = 128, BN = 128;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int BK = 8 * EPC;
  __shared__ u32x4_t lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mat = blockIdx.y;
  int ti, tj;
  if (a.tri) {
    tri_decode(blockIdx.x, ti, tj);
  } else {
    ti = blockIdx.x / a.tiles_n;
    tj = blockIdx.x - ti * a.tiles_n;
  }
  const T* Pm = static_cast<const T*>(a.P) + (long long)mat * a.sP + (long long)ti * BM * a.ldp;
  const T* Qm = static_cast<const T*>(a.Q) + (long long)mat * a.sQ + (long long)tj * BN * a.ldq;

  const int lch = tid & 7, lrow = tid >> 3;
  u32x4_t rp[4], rq[4];
  const int nk = a.K / BK;

  auto gload = [&](int kt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rp[s] = *reinterpret_cast<const u32x4_t*>(Pm + (long long)(lrow + 32 * s) * a.ldp + kt * BK + lch * EPC);
      rq[s] = *reinterpret_cast<const u32x4_t*>(Qm + (long long)(lrow + 32 * s) * a.ldq + kt * BK + lch * EPC);
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = lrow + 32 * s;
      lds[b][r * 8 + (lch ^ (r & 7))] = rp[s];
      lds[b][(BM + r) * 8 + (lch ^ (r & 7))] = rq[s];
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      u32x4_t fa[2], fb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = wm * 64 + mi * 32 + (lane & 31);
        fa[mi] = lds[cur][r * 8 + (ch ^ (r & 7))];
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        fb[ni] = lds[cur][(BM + r) * 8 + (ch ^ (r & 7))];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) mma<T>(acc[mi][ni], fa[mi], fb[ni]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  MFMA 32x32 accumulator layout: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 tile.
  const int i_base = ti * BM + wm * 64, j_base = tj * BN + wn * 64;
  float alpha = 1.f, scl = 1.f;
  if (a.inv) {
    const float v = a.inv[mat];
    alpha = v * v;
    scl = v;
  }
  T* C = static_cast<T*>(a.C) + (long long)mat * a.sC;
  const T* Ain = static_cast<const T*>(a.Ain) + (long long)mat * a.sAin;
  float* Xf = a.Xf + (long long)mat * a.sXf;
  bf16_t* Xb = a.Xb ? static_cast<bf16_t*>(a.Xb) + (long long)mat * a.sXf : nullptr;
  T* XT = static_cast<T*>(a.XTo) + (long long)mat * a.sXT;
  const bool mirror = ti != tj;
  const bool tall = (a.tall_mask >> mat) & 1ull;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i_base + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int j = j_base + ni * 32 + (lane & 31);
        float v = acc[mi][ni][r];
        if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY) {
          if constexpr (EPI == EPI_GRAM) {
            v *= alpha;
          } else {
            v = a.b * to_f32(Ain[(long long)i * a.ldc + j]) + a.c * v;
          }
          const T o = from_f32<T>(v);
          C[(long long)i * a.ldc + j] = o;
          if (mirror) C[(long long)j * a.ldc + i] = o;
        } else {
          const long long o = (long long)i * a.ldx + j;
          const float x = scl * (a.a * Xf[o] + v);
          if (!a.last) {
            Xf[o] = x;
            if (Xb) Xb[o] = from_f32<bf16_t>(x);
            XT[(long long)j * a.ldxt + i] = from_f32<T>(x);
          } else if (i < a.m && j < a.n) {
            const long long oo = tall ? (long long)j * a.m + i : (long long)i * a.n + j;
            if (a.final_mode == FINAL_OUT) {
              if (a.out_bf16)
                static_cast<bf16_t*>(a.out)[(long long)mat * a.s_out + oo] = from_f32<bf16_t>(x);
              else
                static_cast<float*>(a.out)[(long long)mat * a.s_out + oo] = x;
            } else if (a.final_mode == FINAL_WEIGHTS) {
              float* W = wt.w[mat];
              W[oo] = fmaf(a.neg_lr * wt.scale[mat], x, W[oo]);
            }
          }
        }
      }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_prep(int grad_bf16, int compute_bf16, int momentum, const PrepArgs& a,
                       const PrepTable& t, int batch, hipStream_t s) {
  const dim3 grid(a.nblk, batch), block(256);
#define MUON_PREP(GT, CT, MOM) hipLaunchKernelGGL((prep_kernel<GT, CT, MOM>), grid, block, 0, s, a, t)
  if (grad_bf16) {
    if (compute_bf16) {
      if (momentum) MUON_PREP(bf16_t, bf16_t, true); else MUON_PREP(bf16_t, bf16_t, false);
    } else {
      if (momentum) MUON_PREP(bf16_t, float, true); else MUON_PREP(bf16_t, float, false);
    }
  } else {
    if (compute_bf16) {
      if (momentum) MUON_PREP(float, bf16_t, true); else MUON_PREP(float, bf16_t, false);
    } else {
      if (momentum) MUON_PREP(float, float, true); else MUON_PREP(float, float, false);
    }
  }
#undef MUON_PREP
  return hipGetLastError();
}

hipError_t launch_norm(const float* partials, int nblk, float eps, float* inv, int batch,
                       hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(batch), dim3(256), 0, s, partials, nblk, eps, inv);
  return hipGetLastError();
}

hipError_t launch_gemm(int compute_bf16, int epi, const GemmArgs& a, const WeightTable& t,
                       int batch, hipStream_t s) {
  const int tiles = a.tri ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
  const dim3 grid(tiles, batch), block(256);
#define MUON_GEMM(T, E) hipLaunchKernelGGL((gemm_kernel<T, E>), grid, block, 0, s, a, t)
  if (compute_bf16) {
    if (epi == EPI_GRAM) MUON_GEMM(bf16_t, EPI_GRAM);
    else if (epi == EPI_POLY) MUON_GEMM(bf16_t, EPI_POLY);
    else MUON_GEMM(bf16_t, EPI_UPDATE);
  } else {
    if (epi == EPI_GRAM) MUON_GEMM(float, EPI_GRAM);
    else if (epi == EPI_POLY) MUON_GEMM(float, EPI_POLY);
    else MUON_GEMM(float, EPI_UPDATE);
  }
#undef MUON_GEMM
  return hipGetLastError();
}

}  // namespace muon
