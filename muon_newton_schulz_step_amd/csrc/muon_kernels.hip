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
//   gemm_kernel    C[i][j] = sum_k P[i][k] Q[j][k] on MFMA, epilogues:
//                    GRAM   A = X X^T        (lower-triangle tiles, mirrored;
//                                             GRAM_LO: also A's bf16 residual
//                                             on the lower tiles)
//                    POLY   B = b A + c A A  (A symmetric, so A A = A A^T);
//                           the same kernel forms A' = Q A Q, Q = aI + B,
//                           as T = aA + B A (POLY_LO: A with its residual),
//                           then A' = aT + T B
//                    UPDATE X <- a X + B X   (bf16: Q is X's hi plane, read
//                                             row-major and transposed in LDS;
//                                             fp32: Q = X^T, kept as a copy;
//                                             UPDATE_ROWS: also each row's sum
//                                             of X'^2 per 64-column block)
//                    FINAL  the last UPDATE, into the weights (with page 1's
//                           decoupled or cautious weight decay) or the output
//   normuon_rows_kernel  NorMuon (page 1): per oriented row, the mean of O^2,
//                        the second-moment update and the row's scale
//                        (bf16: normuon_rowparts_kernel, from UPDATE_ROWS' sums)
//   apply_kernel         with NorMuon, the weight update as its own pass
// The 1/||u|| normalisation is folded into the first GRAM (x inv^2) and
// UPDATE (x inv) epilogues.
#include "muon_gemm.h"

namespace muon {

// ---------------------------------------------------------------- prep
// One 64x64 tile of the oriented, padded M x N space per block.  Reads the
// original matrix coalesced along its rows; outputs that share the original
// layout are written directly, the others through a transposing LDS tile.
//   CT = bf16: X_0 as its hi plane (bf16) and its lo plane (one byte per
//              element, lo8_of), M x N each;
//   CT = fp32: X_0 (M x N) and X_0^T (N x M).
template <typename GT, typename CT, bool MOM, bool STRM>
__global__ __launch_bounds__(256) void prep_kernel(PrepLaunch launch) {
  const PrepArgs& a = launch.a;
  auto ldx = [](const auto* q) { if constexpr (STRM) return ld_nt(q); else return *q; };
  auto stx = [](auto v, auto* q) { if constexpr (STRM) st_nt(v, q); else *q = v; };
  __shared__ float tile[kPrepTile][kPrepTile + 1];
  __shared__ float red[4];
  constexpr bool HILO = sizeof(CT) == 2;
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
    g = static_cast<const GT*>(kernarg<PrepLaunch>().t.g[mat]);
    buf = kernarg<PrepLaunch>().t.buf[mat];
  } else {
    g = static_cast<const GT*>(a.in) + (long long)mat * a.s_in;
  }
  bf16_t* Xh = nullptr;
  unsigned char* Xl = nullptr;
  float* Xf = nullptr;
  float* XT = nullptr;
  if constexpr (HILO) {
    Xh = static_cast<bf16_t*>(a.Xh) + (long long)mat * a.sX;
    Xl = static_cast<unsigned char*>(a.Xl) + (long long)mat * a.sX;
  } else {
    Xf = a.Xf + (long long)mat * a.sX;
    XT = static_cast<float*>(a.XT) + (long long)mat * a.sXT;
  }
  // X[oi][oj] at offset o.  Every lane of the wave takes part, lane l at
  // o0 + l for one row run of 64 (o0 a multiple of 64): the lo bytes of 4
  // neighbouring lanes go out as one 4-byte store.
  auto put_x = [&](long long o, float u) {
    if constexpr (HILO) {
      const bf16_t hi = from_f32<bf16_t>(u);
      stx(hi, Xh + o);
      const unsigned b = lo8_of(u, to_f32(hi));
      const unsigned w = b | (__shfl_down(b, 1) << 8) | (__shfl_down(b, 2) << 16) |
                         (__shfl_down(b, 3) << 24);
      if ((tid & 3) == 0) stx(w, reinterpret_cast<unsigned*>(Xl + o));
    } else {
      Xf[o] = u;
    }
  };

  const int cc = tid & 63, rr = tid >> 6;
  float sum = 0.f;
#pragma unroll 4
  for (int p = 0; p < kPrepTile / 4; ++p) {
    const int lr = rr + 4 * p;
    const int r = r0 + lr, c = c0 + cc;
    float u = 0.f;
    if (r < rows && c < cols) {
      const long long idx = (long long)r * cols + c;
      const float gv = to_f32(ldx(g + idx));
      if constexpr (MOM) {
        const float nb = a.mu * ldx(buf + idx) + gv;  // buf' = mu*buf + g
        stx(nb, buf + idx);
        u = gv + a.mu * nb;                     // u = g + mu*buf'
      } else {
        u = gv;
      }
    }
    sum += u * u;
    if (!tall) {
      put_x((long long)r * a.N + c, u);  // X[oi][oj] = X[r][c]
    } else if constexpr (!HILO) {
      XT[(long long)r * a.M + c] = u;    // X^T[oj][oi] = X^T[r][c]
    }
    tile[lr][cc] = u;
  }
  __syncthreads();
#pragma unroll 4
  for (int p = 0; p < kPrepTile / 4; ++p) {
    const int lc = rr + 4 * p;
    const float u = tile[cc][lc];
    const int r = r0 + cc, c = c0 + lc;
    if (tall) {
      put_x((long long)c * a.N + r, u);  // X[oi][oj] = X[c][r]
    } else if constexpr (!HILO) {
      XT[(long long)c * a.M + r] = u;    // X^T[oj][oi] = X^T[c][r]
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

// ---------------------------------------------------------------- NorMuon
// One block per oriented row i of the final X (= O) of each matrix: the sum
// of O[i][j]^2 over the row (fixed order: per-thread strided partials, wave
// butterfly, the four waves in order), then the second-moment update and
// the row's scale 1/(sqrt(v') + eps2).  Padding rows (i >= m) get scale 0.
template <bool HILO>
__global__ __launch_bounds__(256) void normuon_rows_kernel(NormuonLaunch launch) {
  const NormuonArgs& a = launch.a;
  __shared__ float red[4];
  const int i = blockIdx.x, mat = blockIdx.y, tid = threadIdx.x;
  const long long row = (long long)mat * a.sX + (long long)i * a.ldx;
  float s = 0.f;
  if constexpr (HILO) {
    const bf16_t* h = static_cast<const bf16_t*>(a.Xh) + row;
    const unsigned char* l = static_cast<const unsigned char*>(a.Xl) + row;
    for (int j = 8 * tid; j < a.N; j += 8 * 256) {
      const bf16x8_t hv = *reinterpret_cast<const bf16x8_t*>(h + j);
      const u32x2_t lv = *reinterpret_cast<const u32x2_t*>(l + j);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = lo8_x(to_f32(hv[e]), lo8_byte(lv[e / 4], e % 4));
        s = fmaf(x, x, s);
      }
    }
  } else {
    const float* f = a.Xf + row;
    for (int j = 4 * tid; j < a.N; j += 4 * 256) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(f + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(v[e], v[e], s);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    float r = 0.f;
    if (i < a.m) {
      const float total = (red[0] + red[1]) + (red[2] + red[3]);
      float* v = kernarg<NormuonLaunch>().t.v[mat];
      const float nv = a.beta2 * v[i] + (1.f - a.beta2) * (total / (float)a.n);
      v[i] = nv;
      r = 1.f / (sqrtf(nv) + a.eps2);
    }
    a.rinv[(long long)mat * a.M + i] = r;
  }
}

// The same from the row sums that the last bf16 UPDATE left per 64-column
// block: one thread per oriented row, the blocks added in column order.
__global__ __launch_bounds__(256) void normuon_rowparts_kernel(NormuonLaunch launch) {
  const NormuonArgs& a = launch.a;
  const int i = blockIdx.x * 256 + threadIdx.x, mat = blockIdx.y;
  const float* p = a.rowpart + (long long)mat * a.s_rp + i;
  const int nb = a.N / 64;
  float total = 0.f;
  for (int jb = 0; jb < nb; ++jb) total += p[(long long)jb * a.ld_rp];
  float r = 0.f;
  if (i < a.m) {
    float* v = kernarg<NormuonLaunch>().t.v[mat];
    const float nv = a.beta2 * v[i] + (1.f - a.beta2) * (total / (float)a.n);
    v[i] = nv;
    r = 1.f / (sqrtf(nv) + a.eps2);
  }
  a.rinv[(long long)mat * a.M + i] = r;
}

// The weight update as its own pass: one 64x64 tile of the oriented, padded
// M x N space per block, like prep_kernel in reverse.  O*rinv[i] is read
// coalesced along the oriented rows; a tall matrix's weights (stored
// transposed to the oriented X) are updated through a transposing LDS tile.
template <bool HILO>
__global__ __launch_bounds__(256) void apply_kernel(ApplyLaunch launch) {
  const ApplyArgs& a = launch.a;
  __shared__ float tile[kPrepTile][kPrepTile + 1];
  const int tid = threadIdx.x, mat = blockIdx.y, bt = blockIdx.x;
  const int oi0 = (bt / a.tiles_n) * kPrepTile;
  const int oj0 = (bt % a.tiles_n) * kPrepTile;
  const bool tall = (a.tall_mask >> mat) & 1ull;
  float* __restrict__ W = kernarg<ApplyLaunch>().wt.w[mat];
  const float wscale = a.neg_lr * kernarg<ApplyLaunch>().wt.scale[mat];
  const float* rinv = a.rinv + (long long)mat * a.M;
  const long long base = (long long)mat * a.sX;
  auto o_at = [&](int oi, int oj) {
    const long long o = base + (long long)oi * a.ldx + oj;
    float x;
    if constexpr (HILO) {
      x = lo8_x(to_f32(ld_nt(static_cast<const bf16_t*>(a.Xh) + o)),
                (int)ld_nt(static_cast<const signed char*>(a.Xl) + o));
    } else {
      x = a.Xf[o];
    }
    return x * rinv[oi];
  };
  const int cc = tid & 63, rr = tid >> 6;
  if (!tall) {
#pragma unroll 4
    for (int p = 0; p < kPrepTile / 4; ++p) {
      const int oi = oi0 + rr + 4 * p, oj = oj0 + cc;  // = original (row, col)
      if (oi < a.m && oj < a.n) {
        const float x = o_at(oi, oj);
        const long long idx = (long long)oi * a.n + oj;
        st_nt(weight_step(ld_nt(W + idx), x, wscale, a.neg_lrwd, a.cautious), W + idx);
      }
    }
  } else {
#pragma unroll 4
    for (int p = 0; p < kPrepTile / 4; ++p) tile[rr + 4 * p][cc] = o_at(oi0 + rr + 4 * p, oj0 + cc);
    __syncthreads();
#pragma unroll 4
    for (int p = 0; p < kPrepTile / 4; ++p) {
      const int lc = rr + 4 * p;
      const int r = oj0 + lc, c = oi0 + cc;  // original (row, col) of oriented (c, r)
      if (r < a.n && c < a.m) {
        const long long idx = (long long)r * a.m + c;
        st_nt(weight_step(ld_nt(W + idx), tile[cc][lc], wscale, a.neg_lrwd, a.cautious), W + idx);
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_prep(int grad_bf16, int compute_bf16, int momentum, const PrepArgs& a,
                       const PrepTable& t, int batch, hipStream_t s) {
  const dim3 grid(a.nblk, batch), block(256);
  const PrepLaunch launch{a, t};
#define MUON_PREP(GT, CT, MOM)                                                      \
  do {                                                                              \
    if (a.stream)                                                                   \
      hipLaunchKernelGGL((prep_kernel<GT, CT, MOM, true>), grid, block, 0, s, launch);  \
    else                                                                            \
      hipLaunchKernelGGL((prep_kernel<GT, CT, MOM, false>), grid, block, 0, s, launch); \
  } while (0)
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

hipError_t launch_normuon_rows(int compute_bf16, const NormuonArgs& a, const RowTable& t,
                               int batch, hipStream_t s) {
  const NormuonLaunch launch{a, t};
  if (compute_bf16 && a.rowpart)
    hipLaunchKernelGGL(normuon_rowparts_kernel, dim3(a.M / 256, batch), dim3(256), 0, s, launch);
  else if (compute_bf16)
    hipLaunchKernelGGL(normuon_rows_kernel<true>, dim3(a.M, batch), dim3(256), 0, s, launch);
  else
    hipLaunchKernelGGL(normuon_rows_kernel<false>, dim3(a.M, batch), dim3(256), 0, s, launch);
  return hipGetLastError();
}

hipError_t launch_apply(int compute_bf16, const ApplyArgs& a, const WeightTable& t, int batch,
                        hipStream_t s) {
  const ApplyLaunch launch{a, t};
  const dim3 grid((a.M / kPrepTile) * a.tiles_n, batch);
  if (compute_bf16)
    hipLaunchKernelGGL(apply_kernel<true>, grid, dim3(256), 0, s, launch);
  else
    hipLaunchKernelGGL(apply_kernel<false>, grid, dim3(256), 0, s, launch);
  return hipGetLastError();
}

int gemm_tile(int compute_bf16, int tile_pref) {
  if (!compute_bf16) return 128;
  return tile_pref == 128 ? 128 : 256;
}

hipError_t launch_gemm(int compute_bf16, int epi, int tile, const GemmArgs& a_in,
                       const WeightTable& t, int batch, hipStream_t s) {
  GemmArgs a = a_in;
  a.tiles_per_mat = a.tri ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
  // grid.y = matrices, grid.x = tiles; the kernel linearises and remaps both
  const dim3 grid(a.tiles_per_mat, batch);
  if (!compute_bf16) {
    // fp32 path: 128 x 128 tiles (the transposed epilogue tile fits in LDS)
    launch_gemm_fp32(epi, a, t, grid, s);
  } else if (epi == EPI_GRAM || epi == EPI_GRAM_LO) {
    launch_gemm_gram(epi, tile, a, t, grid, s);
  } else if (epi == EPI_POLY || epi == EPI_POLY_LO) {
    launch_gemm_poly(epi, tile, a, t, grid, s);
  } else if (epi == EPI_UPDATE || epi == EPI_UPDATE_ROWS) {
    launch_gemm_update(epi, tile, a, t, grid, s);
  } else if (epi == EPI_FINAL_W || epi == EPI_FINAL_W_T || epi == EPI_FINAL_W_MIX) {
    launch_gemm_final_w(epi, tile, a, t, grid, s);
  } else {
    launch_gemm_final_out(epi, tile, a, t, grid, s);
  }
  return hipGetLastError();
}

}  // namespace muon
