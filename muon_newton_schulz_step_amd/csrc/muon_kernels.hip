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

#include <cstdlib>
#include <utility>

#include "muon_kernels.h"

namespace muon {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Kernel arguments are read in place from the kernarg segment: indexing a
// per-matrix table with the matrix index must not copy the table to scratch.
template <typename Arg>
__device__ __forceinline__ const __attribute__((address_space(4))) Arg& kernarg() {
  return *(const __attribute__((address_space(4))) Arg*)__builtin_amdgcn_kernarg_segment_ptr();
}

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

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>), so that
// register arrays are never indexed at run time (which would put them in
// scratch memory).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- prep
// One 64x64 tile of the oriented, padded M x N space per block.  Reads the
// original matrix coalesced along its rows, writes the copy that shares the
// original layout directly and the transposed copy through an LDS tile.
template <typename GT, typename CT, bool MOM>
__global__ __launch_bounds__(256) void prep_kernel(PrepLaunch launch) {
  const PrepArgs& a = launch.a;
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
    g = static_cast<const GT*>(kernarg<PrepLaunch>().t.g[mat]);
    buf = kernarg<PrepLaunch>().t.buf[mat];
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

// Workgroups of a launch are dispatched round-robin over the 8 XCDs
// (workgroup w runs on XCD w % 8, each XCD with its own L2).  Remap so that
// every XCD works through one contiguous range of logical tiles: the tiles
// of one matrix, and neighbouring tiles within it, then share an L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int x = w & 7, k = w >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + k;
}

// Logical tile -> (matrix, tile row, tile column).  Full grids go in groups
// of `group_m` tile rows, column by column, so that the blocks running
// together on an XCD share a few row panels and a few column panels.
__device__ __forceinline__ void decode_tile(const GemmArgs& a, int& mat, int& ti, int& tj) {
  const int total = a.tiles_per_mat * (int)gridDim.y;
  const int L = xcd_remap((int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x, total);
  mat = L / a.tiles_per_mat;
  const int t = L - mat * a.tiles_per_mat;
  if (a.tri) {
    tri_decode(t, ti, tj);
  } else {
    const int span = a.group_m * a.tiles_n;
    const int g = t / span;
    const int first = g * a.group_m;
    const int gm = a.tiles_m - first < a.group_m ? a.tiles_m - first : a.group_m;
    const int idx = t - g * span;
    ti = first + idx % gm;
    tj = idx / gm;
  }
}

// LDS slot of 16-byte chunk `c` of tile row `r`, rows of CPR chunks.  The
// LDS has 64 four-byte banks (256 bytes) and serves 16 lanes of a 16-byte
// access per cycle; 256 / (16 CPR) rows share one bank line, so the chunk
// order is permuted by the index of the row's bank line: 16 consecutive rows
// at one chunk then hit 16 distinct bank groups (MFMA operand reads), and the
// CPR lanes writing one row stay distinct (loader stores).
template <int CPR>
__device__ __forceinline__ int swz(int c, int r) {
  constexpr int RPL = 16 / CPR;  // rows per 256-byte bank line
  return c ^ ((r / RPL) % CPR);
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

// Block tile BM x BN computed by WGM x WGN waves, each owning a
// (BM/WGM) x (BN/WGN) sub-tile of 32x32 MFMA tiles.  K advances 128 bytes
// per row (64 bf16 or 32 fp32) per step through two LDS stages; a row's
// 16-byte chunks are permuted (swz) so that both the stores of the loader
// and the operand reads of the MFMA lanes are free of bank conflicts.  Operand fragments are double-buffered in registers.
//
// Epilogue, one 32-row block of the wave tile at a time: first all of its
// inputs are loaded (C/X values the epilogue combines with), then values
// are computed and stored.  The accumulators hold, per lane, 4 consecutive
// rows i of one column j, so row-major C[i][j] outputs are stored directly
// (consecutive lanes -> consecutive j).  Transposed outputs (the mirrored
// triangle of A and B, the next step's X^T) are staged in LDS as [j][i]
// rows and stored as coalesced 16-byte chunks.
// Wait until at most N vector-memory operations of this wave are in flight
// (other counters untouched): s_waitcnt with vmcnt = N, expcnt = 7,
// lgkmcnt = 15.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel stub
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}

// Workgroup barrier for the direct-to-LDS pipeline, without memory fences:
// a fence would wait for every outstanding load, including the loads of
// later k-tiles that must stay in flight.  It is sufficient here because
// (1) each wave waits (vmcnt) for its own loads of the k-tile about to be
// read before arriving, and LDS has no cache, so the data is in place for
// every wave once all have arrived; (2) a wave's LDS reads of the stage that
// is reloaded next have returned before its MFMAs consumed them.  The
// "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_barrier" ::: "memory");
#endif
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// lds_wave_base + 16 l (lds_wave_base must be the same for the whole wave).
__device__ __forceinline__ void load_lds16(const void* src, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
#endif
}

// Main loop variants (template parameter S):
//  S == 0  operands go global -> registers -> LDS, two LDS stages, the next
//          k-tile's loads in flight while the current one is multiplied;
//  S >= 2  operands go global -> LDS directly (global_load_lds_dwordx4:
//          lane l of a wave writes 16 bytes at the wave's LDS address + 16 l),
//          S LDS stages, loads issued S - 1 k-tiles ahead.
// RB is the bytes of one operand row per k-tile (64 or 128).
template <typename T, int EPI, int BM, int BN, int WGM, int WGN, int S, int RB, bool SCHED = false,
          bool EARLY = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmLaunch launch) {
  const GemmArgs& a = launch.a;
  constexpr int NT = 64 * WGM * WGN, NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = RB / 16;              // chunks per operand row and k-tile
  constexpr int BK = CPR * EPC;             // k per k-tile
  constexpr int KK = CPR / 2;               // MFMA k-substeps per k-tile
  constexpr int ROWS = BM + BN;             // P rows, then Q rows
  constexpr int STAGE = ROWS * CPR;         // 16-byte chunks per stage
  constexpr int NSTAGE = S == 0 ? 2 : S;
  constexpr int TLD = BM + 8;               // row stride of the transposed tile
  constexpr size_t MAIN_BYTES = (size_t)NSTAGE * STAGE * 16;
  constexpr size_t EPI_BYTES = (size_t)BN * TLD * sizeof(T);
  constexpr size_t LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  static_assert(FM * 32 * WGM == BM && FN * 32 * WGN == BN, "wave tiles must be 32-aligned");
  static_assert(S == 0 ? RB == 128 : S >= 2, "register path uses 128-byte rows");
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
  u32x4_t* lds = reinterpret_cast<u32x4_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int mat, ti, tj;
  decode_tile(a, mat, ti, tj);
  const T* __restrict__ Pm =
      static_cast<const T*>(a.P) + (long long)mat * a.sP + (long long)ti * BM * a.ldp;
  const T* __restrict__ Qm =
      static_cast<const T*>(a.Q) + (long long)mat * a.sQ + (long long)tj * BN * a.ldq;
  const int nk = a.K / BK;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int arow = wm * WTM + (lane & 31), brow = BM + wn * WTN + (lane & 31);
  const int hsel = lane >> 5;
  u32x4_t fa[2][FM], fb[2][FN];
  auto fload = [&](const u32x4_t* L, int kk, int slot) {
    const int ch = 2 * kk + hsel;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
      const int r = arow + mi * 32;
      fa[slot][mi] = L[r * CPR + swz<CPR>(ch, r)];
    }
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      const int r = brow + ni * 32;
      fb[slot][ni] = L[r * CPR + swz<CPR>(ch, r)];
    }
  };
  auto compute = [&](const u32x4_t* L) {
    fload(L, 0, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) fload(L, kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) mma<T>(acc[mi][ni], fa[kk & 1][mi], fb[kk & 1][ni]);
    }
    if constexpr (S >= 2 && SCHED) {
      // Pinned order: the first substep's reads, then each later substep's
      // reads one after each MFMA of the substep before it.
      __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) {
#pragma unroll
        for (int x = 0; x < FM + FN; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
    }
  };

  if constexpr (S == 0) {
    constexpr int RPP = NT / 8;  // rows per loader pass
    constexpr int PA = BM / RPP, PB = BN / RPP;
    static_assert(PA * RPP == BM && PB * RPP == BN, "tile rows must split over the loader");
    const int lch = tid & 7, lrow = tid >> 3;
    u32x4_t rp[PA], rq[PB];
    auto gload = [&](int kt) {
      const int kofs = kt * BK + lch * EPC;
#pragma unroll
      for (int s = 0; s < PA; ++s)
        rp[s] = *reinterpret_cast<const u32x4_t*>(Pm + (long long)(lrow + RPP * s) * a.ldp + kofs);
#pragma unroll
      for (int s = 0; s < PB; ++s)
        rq[s] = *reinterpret_cast<const u32x4_t*>(Qm + (long long)(lrow + RPP * s) * a.ldq + kofs);
    };
    auto lstore = [&](int b) {
      u32x4_t* L = lds + b * STAGE;
#pragma unroll
      for (int s = 0; s < PA; ++s) {
        const int r = lrow + RPP * s;
        L[r * 8 + swz<8>(lch, r)] = rp[s];
      }
#pragma unroll
      for (int s = 0; s < PB; ++s) {
        const int r = BM + lrow + RPP * s;
        L[r * 8 + swz<8>(lch, r)] = rq[s];
      }
    };
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      compute(lds + cur * STAGE);
      if (kt + 1 < nk) lstore(cur ^ 1);
      __syncthreads();
    }
  } else if constexpr (EARLY) {
    // Two stages, direct-to-LDS loads, and the hand-over between them one
    // k-substep before the end of a k-tile: after the last substep's
    // operands are in registers, the waves meet, the k-tile after next is
    // issued into the stage just finished, and the next k-tile's first
    // operands are read while the last substep's MFMAs run.  The body has
    // no branch: the final two iterations reload the last k-tile into a
    // stage nobody reads any more (drained before the epilogue).
    static_assert(S == 2, "hand-over variant uses two stages");
    constexpr int RPI = 1024 / RB;
    constexpr int DPW = ROWS / RPI / NW;
    static_assert(DPW * RPI * NW == ROWS, "stage rows must split over the waves");
    const T* src[DPW];
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int r = (wave * DPW + d) * RPI + lane / CPR;
      const int c = swz<CPR>(lane % CPR, r);
      src[d] = r < BM ? Pm + (long long)r * a.ldp + c * EPC
                      : Qm + (long long)(r - BM) * a.ldq + c * EPC;
    }
    auto issue = [&](int kt, int stage) {
#pragma unroll
      for (int d = 0; d < DPW; ++d)
        load_lds16(src[d] + (long long)kt * BK,
                   smem + (size_t)stage * STAGE * 16 + (size_t)(wave * DPW + d) * 1024);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) mma<T>(acc[mi][ni], fa[slot][mi], fb[slot][ni]);
    };
    issue(0, 0);
    wait_vmcnt<0>();
    barrier_no_fence();
    issue(nk > 1 ? 1 : 0, 1);
    fload(lds, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const u32x4_t* L = lds + (kt & 1) * STAGE;
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) {
        fload(L, kk + 1, (kk + 1) & 1);
        mfmas(kk & 1);
      }
      if constexpr (SCHED) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
#pragma unroll
          for (int x = 0; x < FM + FN; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
        }
      }
      wait_vmcnt<0>();    // this wave's part of k-tile kt+1 has landed
      barrier_no_fence();  // everyone's has; everyone is done reading stage kt&1
      issue(kt + 2 < nk ? kt + 2 : nk - 1, kt & 1);
      fload(lds + ((kt + 1) & 1) * STAGE, 0, 0);
      mfmas((KK - 1) & 1);
      if constexpr (SCHED) {
        __builtin_amdgcn_sched_group_barrier(0x020, DPW, 0);  // the loads
#pragma unroll
        for (int x = 0; x < FM + FN; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  } else {
    // Direct-to-LDS loads.  One instruction moves 64 x 16 bytes = RPI rows;
    // each wave owns DPW of them per stage.  Lane l fills LDS slot l % CPR of
    // row l / CPR, so it fetches the global chunk that the swizzle puts there.
    constexpr int RPI = 1024 / RB;
    constexpr int DPW = ROWS / RPI / NW;
    static_assert(DPW * RPI * NW == ROWS, "stage rows must split over the waves");
    static_assert(DPW * (S - 2) < 64, "vmcnt range");
    const T* src[DPW];
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int r = (wave * DPW + d) * RPI + lane / CPR;
      const int c = swz<CPR>(lane % CPR, r);
      src[d] = r < BM ? Pm + (long long)r * a.ldp + c * EPC
                      : Qm + (long long)(r - BM) * a.ldq + c * EPC;
    }
    auto issue = [&](int kt, int stage) {
#pragma unroll
      for (int d = 0; d < DPW; ++d)
        load_lds16(src[d] + (long long)kt * BK,
                   smem + (size_t)stage * STAGE * 16 + (size_t)(wave * DPW + d) * 1024);
    };
#pragma unroll
    for (int t = 0; t < S - 1; ++t)
      if (t < nk) issue(t, t);
    for (int kt0 = 0; kt0 < nk; kt0 += S) {
      static_for<S>([&](auto st) {
        const int kt = kt0 + st;
        if (kt < nk) {
          // this wave's loads of k-tile kt have landed once at most
          // min(S - 2, k-tiles issued after it) load groups are in flight
          const int later = nk - 1 - kt;
          if (later >= S - 2) {
            wait_vmcnt<DPW * (S - 2)>();
          } else {
            static_for<S - 2>([&](auto q) {
              if (later == q) wait_vmcnt<DPW * q>();
            });
          }
          barrier_no_fence();  // every wave's loads of kt are in LDS; stage kt-1 is free
          if (kt + S - 1 < nk) issue(kt + S - 1, (st + S - 1) % S);
          compute(lds + st * STAGE);
        }
      });
    }
    __syncthreads();
  }

  // ---- epilogue (LDS is free: the last iteration ended with a barrier)
  const int i_base = ti * BM + wm * WTM, j_base = tj * BN + wn * WTN;
  float alpha = 1.f, scl = 1.f;
  if (a.inv) {
    const float v = a.inv[mat];
    alpha = v * v;
    scl = v;
  }
  const bool tall = (a.tall_mask >> mat) & 1ull;
  // Transposed output of this block: the mirrored tile (GRAM, POLY off the
  // diagonal) or the next step's X^T (UPDATE).
  constexpr bool FINAL = EPI == EPI_FINAL_W || EPI == EPI_FINAL_OUT;
  bool stage_t = false;
  if constexpr (EPI == EPI_UPDATE) stage_t = true;
  if constexpr (EPI == EPI_GRAM || EPI == EPI_POLY) stage_t = ti != tj;
  T* __restrict__ Ts = reinterpret_cast<T*>(smem);
  T* __restrict__ C = nullptr;
  const T* __restrict__ Ain = nullptr;
  float* __restrict__ Xf = nullptr;
  bf16_t* __restrict__ Xb = nullptr;
  float* __restrict__ W = nullptr;
  float wscale = 0.f;
  if constexpr (EPI == EPI_UPDATE || FINAL) {
    Xf = a.Xf + (long long)mat * a.sXf;
    if (a.Xb) Xb = static_cast<bf16_t*>(a.Xb) + (long long)mat * a.sXf;
    if constexpr (EPI == EPI_FINAL_W) {
      W = kernarg<GemmLaunch>().wt.w[mat];
      wscale = a.neg_lr * kernarg<GemmLaunch>().wt.scale[mat];
    }
  } else {
    C = static_cast<T*>(a.C) + (long long)mat * a.sC;
    if constexpr (EPI == EPI_POLY) Ain = static_cast<const T*>(a.Ain) + (long long)mat * a.sAin;
  }
  const int jl0 = wn * WTN + (lane & 31);

  static_for<FM>([&](auto mi) {
    const int ib = i_base + mi * 32 + 4 * hsel;  // + 8q + t
    // phase 1: the inputs of this 32-row block
    float ein[FN][16];
    float win[EPI == EPI_FINAL_W ? FN : 1][16];
    static_for<FN>([&](auto ni) {
      const int j = j_base + ni * 32 + (lane & 31);
      static_for<16>([&](auto r) {
        const int i = ib + 8 * (r / 4) + (r % 4);
        if constexpr (EPI == EPI_POLY) ein[ni][r] = to_f32(Ain[(long long)i * a.ldc + j]);
        if constexpr (EPI == EPI_UPDATE || FINAL) ein[ni][r] = Xf[(long long)i * a.ldx + j];
        if constexpr (EPI == EPI_FINAL_W) {
          // outside the matrix (zero padding) read element 0 and discard it
          const bool inb = i < a.m && j < a.n;
          const long long oo = tall ? (long long)j * a.m + i : (long long)i * a.n + j;
          win[ni][r] = W[inb ? oo : 0];
        }
      });
    });
    // phase 2: values, direct stores, transposed staging
    static_for<FN>([&](auto ni) {
      const int j = j_base + ni * 32 + (lane & 31);
      static_for<4>([&](auto q) {
        float v[4];
        static_for<4>([&](auto t) {
          constexpr int r = 4 * q + t;
          const int i = ib + 8 * q + t;
          const float accv = acc[mi][ni][r];
          if constexpr (EPI == EPI_GRAM) {
            v[t] = accv * alpha;
            C[(long long)i * a.ldc + j] = from_f32<T>(v[t]);
          } else if constexpr (EPI == EPI_POLY) {
            v[t] = a.b * ein[ni][r] + a.c * accv;
            C[(long long)i * a.ldc + j] = from_f32<T>(v[t]);
          } else if constexpr (EPI == EPI_UPDATE) {
            v[t] = scl * (a.a * ein[ni][r] + accv);
            const long long o = (long long)i * a.ldx + j;
            Xf[o] = v[t];
            if (Xb) Xb[o] = from_f32<bf16_t>(v[t]);
          } else {  // FINAL_W, FINAL_OUT
            const float x = scl * (a.a * ein[ni][r] + accv);
            if (i < a.m && j < a.n) {
              const long long oo = tall ? (long long)j * a.m + i : (long long)i * a.n + j;
              if constexpr (EPI == EPI_FINAL_W) {
                W[oo] = fmaf(wscale, x, win[ni][r]);
              } else if (a.out_bf16) {
                static_cast<bf16_t*>(a.out)[(long long)mat * a.s_out + oo] = from_f32<bf16_t>(x);
              } else {
                static_cast<float*>(a.out)[(long long)mat * a.s_out + oo] = x;
              }
            }
          }
        });
        if constexpr (!FINAL) {
          if (stage_t) {
            const int il = wm * WTM + mi * 32 + 8 * q + 4 * hsel, jl = jl0 + ni * 32;
            if constexpr (sizeof(T) == 2) {
              uint2 pk;
              pk.x = (unsigned)__builtin_bit_cast(unsigned short, from_f32<T>(v[0])) |
                     ((unsigned)__builtin_bit_cast(unsigned short, from_f32<T>(v[1])) << 16);
              pk.y = (unsigned)__builtin_bit_cast(unsigned short, from_f32<T>(v[2])) |
                     ((unsigned)__builtin_bit_cast(unsigned short, from_f32<T>(v[3])) << 16);
              *reinterpret_cast<uint2*>(Ts + jl * TLD + il) = pk;
            } else {
              f32x4_t f;
              f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
              *reinterpret_cast<f32x4_t*>(Ts + jl * TLD + il) = f;
            }
          }
        }
      });
    });
  });
  if constexpr (!FINAL) {
    if (stage_t) {
      __syncthreads();
      T* __restrict__ dst;
      int ld;
      if constexpr (EPI == EPI_UPDATE) {
        dst = static_cast<T*>(a.XTo) + (long long)mat * a.sXT;
        ld = a.ldxt;
      } else {
        dst = C;
        ld = a.ldc;
      }
      constexpr int CPR = BM / EPC;  // 16-byte chunks per transposed row
#pragma unroll 4
      for (int c = tid; c < BN * CPR; c += NT) {
        const int jl = c / CPR, il = (c % CPR) * EPC;
        *reinterpret_cast<u32x4_t*>(dst + (long long)(tj * BN + jl) * ld + ti * BM + il) =
            *reinterpret_cast<const u32x4_t*>(Ts + jl * TLD + il);
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_prep(int grad_bf16, int compute_bf16, int momentum, const PrepArgs& a,
                       const PrepTable& t, int batch, hipStream_t s) {
  const dim3 grid(a.nblk, batch), block(256);
  const PrepLaunch launch{a, t};
#define MUON_PREP(GT, CT, MOM) hipLaunchKernelGGL((prep_kernel<GT, CT, MOM>), grid, block, 0, s, launch)
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

int gemm_tile(int compute_bf16, int tile_pref) {
  if (!compute_bf16) return 128;
  return tile_pref == 128 ? 128 : 256;
}

// bf16 256x256 tiles on 8 waves (2x4, 128x64 each).  Main loop, chosen by
// MUON_WAVE_CFG (a tuning knob; by default 5 for GRAM / POLY, 4 otherwise):
//   0  register-staged loads, 128-byte rows, two LDS stages
//   1  direct-to-LDS loads, 64-byte rows, 3 stages
//   3  as 1 with the MFMA / LDS-read order pinned
//   4  direct-to-LDS loads, 128-byte rows, 2 stages, order pinned
//   5  as 4 with the stage hand-over one k-substep before the tile's end
// 128x128 tiles use 4 waves (64x64 each) and register-staged loads.
static int wave_cfg(int epi) {
  static const int v = [] {
    const char* e = std::getenv("MUON_WAVE_CFG");
    return e ? std::atoi(e) : -1;
  }();
  if (v >= 0) return v;
  return epi == EPI_GRAM || epi == EPI_POLY ? 5 : 4;
}

template <typename T, int E>
static void launch_gemm_t(int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                          hipStream_t s) {
  const GemmLaunch launch{a, t};
  if constexpr (sizeof(T) == 2) {
    if (tile == 256) {
      switch (wave_cfg(E)) {
        case 0:
          hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 0, 128>), grid, dim3(512), 0, s,
                             launch);
          return;
        case 1:
          hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 3, 64>), grid, dim3(512), 0, s,
                             launch);
          return;
        case 3:
          hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 3, 64, true>), grid, dim3(512), 0,
                             s, launch);
          return;
        case 5:
          hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 2, 128, true, true>), grid,
                             dim3(512), 0, s, launch);
          return;
        default:
          hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 2, 128, true>), grid, dim3(512), 0,
                             s, launch);
          return;
      }
    }
  }
  hipLaunchKernelGGL((gemm_kernel<T, E, 128, 128, 2, 2, 0, 128>), grid, dim3(256), 0, s, launch);
}

hipError_t launch_gemm(int compute_bf16, int epi, int tile, const GemmArgs& a_in,
                       const WeightTable& t, int batch, hipStream_t s) {
  GemmArgs a = a_in;
  a.tiles_per_mat = a.tri ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
  // grid.y = matrices, grid.x = tiles; the kernel linearises and remaps both
  const dim3 grid(a.tiles_per_mat, batch);
  if (compute_bf16) {
    if (epi == EPI_GRAM) launch_gemm_t<bf16_t, EPI_GRAM>(tile, a, t, grid, s);
    else if (epi == EPI_POLY) launch_gemm_t<bf16_t, EPI_POLY>(tile, a, t, grid, s);
    else if (epi == EPI_UPDATE) launch_gemm_t<bf16_t, EPI_UPDATE>(tile, a, t, grid, s);
    else if (epi == EPI_FINAL_W) launch_gemm_t<bf16_t, EPI_FINAL_W>(tile, a, t, grid, s);
    else launch_gemm_t<bf16_t, EPI_FINAL_OUT>(tile, a, t, grid, s);
  } else {
    // fp32 path: 128 x 128 tiles (the transposed epilogue tile fits in LDS)
    if (epi == EPI_GRAM) launch_gemm_t<float, EPI_GRAM>(128, a, t, grid, s);
    else if (epi == EPI_POLY) launch_gemm_t<float, EPI_POLY>(128, a, t, grid, s);
    else if (epi == EPI_UPDATE) launch_gemm_t<float, EPI_UPDATE>(128, a, t, grid, s);
    else if (epi == EPI_FINAL_W) launch_gemm_t<float, EPI_FINAL_W>(128, a, t, grid, s);
    else launch_gemm_t<float, EPI_FINAL_OUT>(128, a, t, grid, s);
  }
  return hipGetLastError();
}

}  // namespace muon
