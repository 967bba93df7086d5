// The batched MFMA GEMM of the Newton-Schulz steps (gemm_kernel) and its
// launcher template.  Each epilogue family is instantiated in a translation
// unit of its own (gemm_*.hip), so that they compile in parallel.
// Internal; not part of the C ABI.
#pragma once

#include "muon_device.h"

namespace muon {

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
  const int lm = L / a.tiles_per_mat;
  const int t = L - lm * a.tiles_per_mat;
  mat = a.mat0 + lm;
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

// LDS slot of 16-byte chunk `c` of a 128-byte operand row `r`.  The LDS has
// 64 four-byte banks (256 bytes per bank line) and serves 16 lanes of a
// 16-byte access per cycle; two rows share a bank line, so the chunk order
// is permuted by the row pair index: 16 consecutive rows at one chunk hit 16
// distinct bank groups (MFMA operand reads), and the 8 lanes filling one row
// stay distinct.  An involution: slot s of row r holds chunk swz(s, r).
__device__ __forceinline__ int swz(int c, int r) { return c ^ ((r >> 1) & 7); }

// Row-major [k][j] operand tile (bf16 UPDATE's X), k-rows of SEGS 64-byte
// segments (4 chunks each): the segment order of k-row k is permuted by
// k % SEGS.  A transposing read touches 4 consecutive k-rows at one logical
// segment per 32 lanes, which then fall on 4 distinct quarters of the bank
// line.  Also an involution, in the chunk index u.
template <int SEGS>
__device__ __forceinline__ int qrow_unit(int k, int u) {
  return (((u >> 2) ^ (k % SEGS)) << 2) | (u & 3);
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

// Wait until this wave has no vector-memory operation and no LDS operation in
// flight: s_waitcnt vmcnt(0) lgkmcnt(0) (expcnt untouched).
__device__ __forceinline__ void wait_vm_lgkm0() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((7 << 4));
#endif
}

// Workgroup barrier for the direct-to-LDS pipeline, without memory fences:
// a fence would wait for every outstanding load, including the loads of
// later k-tiles that must stay in flight.  It is sufficient here because,
// before arriving, each wave waits (wait_vm_lgkm0) for (1) its own loads of
// the k-tile about to be read (LDS has no cache, so the data is in place for
// every wave once all have arrived) and (2) its own LDS reads of the stage
// that the waves refill right after the barrier: an LDS read still queued
// when another wave's direct-to-LDS load lands would return the next
// k-tile's data.  The "memory" clobber keeps the compiler from moving LDS
// accesses across it.
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

// The same 16-byte direct-to-LDS load through a buffer resource (MUBUF).
// A global (FLAT-encoded) load that writes LDS counts as pending on both the
// vector-memory and the LDS counters, which forces every LDS wait behind it
// to drain all LDS reads (lgkmcnt(0)); the buffer form counts on vmcnt only.
// Buffer resource word 3 on gfx9-family chips: 32-bit data format, no
// swizzle; stride 0 (raw), range 0xffffffff (no range clamping).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)0xffffffff,
                                           0x00020000);
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset,
                                                  void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, (int)voffset, 0, 0, 0);
#endif
}

// Transposing LDS read of 4 x 16 bits (ds_read_b64_tr_b16), 8-byte aligned
// addresses.  In each group of 16 lanes, lane i receives element i % 4 of
// the 8-byte rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12, in
// that order.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
#else
  return u32x2_t{0u, 0u};
#endif
}

// Block tile BM x BN computed by WGM x WGN waves, each owning a
// (BM/WGM) x (BN/WGN) sub-tile of 32x32 MFMA tiles, fp32 accumulators.  K
// advances 128 bytes per operand row (64 bf16 or 32 fp32) per k-tile.
//
// A stage holds the k-tile of both operands in 16-byte chunks: BM rows of P
// (8 chunks each, swz), then Q's BN rows (8 chunks each, swz) or, with QROW,
// Q's row-major k-tile: BK k-rows of BN / 8 chunks (qrow_unit), read with
// the transposing LDS read, which hands each lane 4 k-values of its column.
//
// Main loop (S):
//   S == 0  global -> registers -> LDS, two stages, the next k-tile's loads in
//           flight while the current one is multiplied (the fp32 path);
//   S == 2  global -> LDS directly, two stages, an explicit vmcnt wait and a
//           fence-free barrier per k-tile, one k-substep before the k-tile's
//           end; the order of MFMAs and operand reads is pinned (each later
//           k-substep's reads go one after each MFMA of the substep before).
//           BUFLD: buffer (MUBUF) loads, else global (FLAT) ones.
//
// Epilogue, one 32-row block of the wave tile at a time: inputs loaded first,
// then values computed and stored.  The accumulators hold, per lane, 4
// consecutive rows i of one column j, so row-major outputs can be stored
// directly (consecutive lanes -> consecutive j): GRAM, POLY and the FINAL of
// wide matrices do so.  The bf16 UPDATE instead stages each block as fp32
// rows in LDS and moves X in 16-byte runs of 8 columns; transposed outputs
// (the mirrored triangle of A and B, the fp32 path's X^T, the weights of a
// tall matrix) are staged in LDS as [j][i] rows and stored as coalesced
// 16-byte chunks.
template <typename T, int EPI, int BM, int BN, int WGM, int WGN, int S, bool QROW, bool BUFLD,
          bool STRM>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmLaunch launch) {
  const GemmArgs& a = launch.a;
  // STRM: the X state and the weights are streamed (see ld_nt)
  auto ldx = [](const auto* q) { if constexpr (STRM) return ld_nt(q); else return *q; };
  auto stx = [](auto v, auto* q) { if constexpr (STRM) st_nt(v, q); else *q = v; };
  constexpr bool SCHED = S == 2;
  constexpr int NT = 64 * WGM * WGN, NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = 8;                    // chunks per operand row and k-tile
  constexpr int BK = CPR * EPC;             // k per k-tile
  constexpr int KK = 4;                     // MFMA k-substeps per k-tile
  constexpr int P_CHUNKS = BM * CPR;
  constexpr int STAGE = P_CHUNKS + BN * CPR;  // with QROW: BK * (BN / 8), the same
  constexpr int UPR = BN / 8;                 // QROW: chunks per k-row
  constexpr int SEGS = BN / 32;               // QROW: 64-byte segments per k-row
  constexpr int TLD = BM + 8;                 // row stride of the transposed tile
  constexpr size_t MAIN_BYTES = 2 * (size_t)STAGE * 16;
  constexpr size_t EPI_BYTES = (size_t)BN * TLD * sizeof(T);
  constexpr size_t LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  constexpr bool FIN_W = EPI == EPI_FINAL_W || EPI == EPI_FINAL_W_T || EPI == EPI_FINAL_W_MIX;
  constexpr bool FIN_OUT = EPI == EPI_FINAL_OUT || EPI == EPI_FINAL_OUT_T;
  constexpr bool FINAL = FIN_W || FIN_OUT;
  constexpr bool TALLF = EPI == EPI_FINAL_W_T || EPI == EPI_FINAL_OUT_T;  // FINAL, tall matrices
  constexpr bool MIXF = EPI == EPI_FINAL_W_MIX;  // FINAL, the orientation per matrix
  constexpr bool HILO = sizeof(T) == 2;  // bf16 path: X state as hi + lo planes
  constexpr bool GRAMK = EPI == EPI_GRAM || EPI == EPI_GRAM_LO;
  constexpr bool POLYK = EPI == EPI_POLY || EPI == EPI_POLY_LO;
  constexpr bool UPD = EPI == EPI_UPDATE || EPI == EPI_UPDATE_ROWS;
  constexpr bool ROWS = EPI == EPI_UPDATE_ROWS;
  static_assert(!ROWS || HILO, "row sums on the bf16 path");
  static_assert(!MIXF || HILO, "mixed orientations on the bf16 path");
  constexpr bool STAGED_T = GRAMK || POLYK || (UPD && !HILO);
  static_assert(FM * 32 * WGM == BM && FN * 32 * WGN == BN, "wave tiles must be 32-aligned");
  static_assert(S == 0 || S == 2, "main loop variants");
  static_assert(!QROW || (HILO && BK == 64 && !STAGED_T), "row-major Q is the bf16 X operand");
  // The two stages.  With QROW they are two distinct LDS objects: the
  // compiler's wait analysis then sees that the transposing reads of one
  // stage do not alias the direct-to-LDS loads in flight into the other
  // (with one object it waits for every load before each such read).  The
  // QROW epilogues stage nothing in LDS.  Otherwise one object holds both
  // stages and, in the epilogue, the transposed tile.
  u32x4_t* S0;
  u32x4_t* S1;
  unsigned char* smem;
  if constexpr (QROW) {
    __shared__ u32x4_t stage0[STAGE], stage1[STAGE];
    S0 = stage0;
    S1 = stage1;
    smem = nullptr;
  } else {
    __shared__ __attribute__((aligned(16))) unsigned char lds_all[LDS_BYTES];
    smem = lds_all;
    S0 = reinterpret_cast<u32x4_t*>(lds_all);
    S1 = S0 + STAGE;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int mat, ti, tj;
  decode_tile(a, mat, ti, tj);
  const T* __restrict__ Pm =
      static_cast<const T*>(a.P) + (long long)mat * a.sP + (long long)ti * BM * a.ldp;
  // Q's tile: BN rows from row tj * BN, or (QROW) BN columns from column tj * BN
  const T* __restrict__ Qm =
      QROW ? static_cast<const T*>(a.Q) + (long long)mat * a.sQ + (long long)tj * BN
           : static_cast<const T*>(a.Q) + (long long)mat * a.sQ + (long long)tj * BN * a.ldq;
  const int nk = a.K / BK;
  // Advance of a Q chunk's source per k-tile, in elements (P's is BK).
  const long long qstep = QROW ? (long long)BK * a.ldq : BK;

  // Global source, at k-tile 0, of the chunk that fills LDS chunk q of a stage.
  auto chunk_src = [&](int q) -> const T* {
    if (q < P_CHUNKS) {
      const int r = q / CPR;
      return Pm + (long long)r * a.ldp + swz(q % CPR, r) * EPC;
    }
    const int qq = q - P_CHUNKS;
    if constexpr (QROW) {
      const int k = qq / UPR;
      return Qm + (long long)k * a.ldq + qrow_unit<SEGS>(k, qq % UPR) * EPC;
    } else {
      const int r = qq / CPR;
      return Qm + (long long)r * a.ldq + swz(qq % CPR, BM + r) * EPC;
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  const int arow = wm * WTM + (lane & 31), brow = BM + wn * WTN + (lane & 31);
  const int hsel = lane >> 5;
  // QROW operand reads: lane c of a 16-lane group addresses k-row
  // 16 kk + 8 hsel + 4 h + c / 4 and columns j .. j + 3, j = 16 g + 4 (c % 4)
  // within its 32-column block (g = the group's position in its half-wave),
  // so lane (32 hsel + 16 g + c) receives column 16 g + c, k = 8 hsel + 4 h + e.
  const int tr_k = 8 * hsel + ((lane & 15) >> 2);
  const int tr_j = wn * WTN + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  u32x4_t fa[2][FM], fb[2][FN];
  // Operand reads of k-substep kk in the order the MFMAs (mi-major) first
  // use them: A row block 0, every B column block, then the other A blocks.
  auto fload = [&](const u32x4_t* L, int kk, int slot) {
    const int ch = 2 * kk + hsel;
    auto read_a = [&](int mi) {
      const int r = arow + mi * 32;
      fa[slot][mi] = L[r * CPR + swz(ch, r)];
    };
    read_a(0);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
      if constexpr (QROW) {
        const unsigned char* Lq = reinterpret_cast<const unsigned char*>(L + P_CHUNKS);
        const int j = tr_j + ni * 32;
        u32x2_t half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = 16 * kk + tr_k + 4 * h;
          half[h] = lds_read_tr16(Lq + (k * UPR + qrow_unit<SEGS>(k, j >> 3)) * 16 + (j & 7) * 2);
        }
        fb[slot][ni] = u32x4_t{half[0][0], half[0][1], half[1][0], half[1][1]};
      } else {
        const int r = brow + ni * 32;
        fb[slot][ni] = L[r * CPR + swz(ch, r)];
      }
    }
#pragma unroll
    for (int mi = 1; mi < FM; ++mi) read_a(mi);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) mma<T>(acc[mi][ni], fa[slot][mi], fb[slot][ni]);
  };
  // LDS reads per k-substep, and the pinned order for n substeps: each
  // MFMA followed by one read of the next substep's operands.
  constexpr int NREAD = FM + (QROW ? 2 * FN : FN);
  constexpr int NPAIR = NREAD < FM * FN ? NREAD : FM * FN;
  auto schedule_substeps = [&](int n) {
    if constexpr (SCHED) {
      for (int kk = 0; kk < n; ++kk) {
#pragma unroll
        for (int x = 0; x < NPAIR; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        if constexpr (FM * FN > NPAIR)
          __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - NPAIR, 0);
        if constexpr (NREAD > NPAIR)
          __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NPAIR, 0);
      }
    }
  };
  auto compute = [&](const u32x4_t* L) {
    fload(L, 0, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) fload(L, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
    }
    if constexpr (SCHED) {
      __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
      schedule_substeps(KK - 1);
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
    }
  };

  // nk is even (K is a multiple of 256), so the k-loops below go two
  // k-tiles per iteration, stage S0 then stage S1, both fixed at compile time.
  if constexpr (S == 0) {
    // Thread t moves LDS chunks t + NT i of each stage.
    constexpr int PER = STAGE / NT;
    static_assert(PER * NT == STAGE && P_CHUNKS % NT == 0, "stage chunks must split over the threads");
    const T* src[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) src[i] = chunk_src(tid + NT * i);
    u32x4_t rg[PER];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const long long step = i < P_CHUNKS / NT ? (long long)BK : qstep;
        rg[i] = *reinterpret_cast<const u32x4_t*>(src[i] + kt * step);
      }
    };
    auto lstore = [&](u32x4_t* St) {
#pragma unroll
      for (int i = 0; i < PER; ++i) St[tid + NT * i] = rg[i];
    };
    auto ktile = [&](int kt, const u32x4_t* cur, u32x4_t* nxt) {
      if (kt + 1 < nk) gload(kt + 1);
      compute(cur);
      if (kt + 1 < nk) lstore(nxt);
      __syncthreads();
    };
    gload(0);
    lstore(S0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      ktile(kt, S0, S1);
      ktile(kt + 1, S1, S0);
    }
  } else {
    // Direct-to-LDS loads: instruction d of wave w moves LDS chunks
    // 64 g .. 64 g + 63 of a stage, g = w DPW + d (lane l: chunk 64 g + l).
    // A wave's chunks all belong to one operand, so its k-tile advance is
    // one wave-uniform value.
    constexpr int DPW = STAGE / 64 / NW;
    static_assert(DPW * 64 * NW == STAGE && P_CHUNKS % (DPW * 64) == 0,
                  "stage chunks must split over the waves, one operand per wave");
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const long long kstep = wave_s * DPW * 64 < P_CHUNKS ? (long long)BK : qstep;
    const T* src[DPW];
#pragma unroll
    for (int d = 0; d < DPW; ++d) src[d] = chunk_src((wave * DPW + d) * 64 + lane);
    // BUFLD: the wave's operand panel as a buffer resource, rebased per k-tile,
    // and 32-bit lane offsets into it (the host checks that they fit)
    const T* wbase = wave_s * DPW * 64 < P_CHUNKS ? Pm : Qm;
    unsigned voff[BUFLD ? DPW : 1];
    if constexpr (BUFLD) {
#pragma unroll
      for (int d = 0; d < DPW; ++d) voff[d] = (unsigned)((src[d] - wbase) * (long long)sizeof(T));
    }
    // loads d0 .. d1 - 1 of k-tile kt into stage St
    auto issue = [&](int kt, u32x4_t* St) {
      const long long off = kt * kstep;
      if constexpr (BUFLD) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(wbase + off);
#pragma unroll
        for (int d = 0; d < DPW; ++d) buffer_load_lds16(rs, voff[d], St + (wave_s * DPW + d) * 64);
      } else {
#pragma unroll
        for (int d = 0; d < DPW; ++d) load_lds16(src[d] + off, St + (wave_s * DPW + d) * 64);
      }
    };
    // The waves meet once the last k-substep's operands are in registers;
    // the k-tile after next then goes into the stage just finished, and the
    // next k-tile's first operands are read while the last substep's MFMAs
    // run.  No branch in the body: the final two k-tiles reload the last
    // k-tile into a stage nobody reads any more (drained below).
    auto ktile = [&](int kt, u32x4_t* cur, const u32x4_t* nxt) {
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) {
        fload(cur, kk + 1, (kk + 1) & 1);
        mfmas(kk & 1);
      }
      schedule_substeps(KK - 1);
      wait_vm_lgkm0();     // this wave's part of k-tile kt+1 has landed and
                           // its reads of cur have returned
      barrier_no_fence();  // everyone's has: cur may be refilled
      issue(kt + 2 < nk ? kt + 2 : nk - 1, cur);
      fload(nxt, 0, 0);
      mfmas((KK - 1) & 1);
      __builtin_amdgcn_sched_group_barrier(0x020, DPW, 0);  // the loads
      schedule_substeps(1);
    };
    issue(0, S0);
    wait_vmcnt<0>();
    barrier_no_fence();
    issue(nk > 1 ? 1 : 0, S1);
    fload(S0, 0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
      ktile(kt, S0, S1);
      ktile(kt + 1, S1, S0);
    }
    wait_vmcnt<0>();
    __syncthreads();
  }

  // ---- epilogue (LDS is free: the main loop ended with a barrier)
  const int i_base = ti * BM + wm * WTM, j_base = tj * BN + wn * WTN;
  float alpha = 1.f, scl = 1.f;
  if (a.inv) {
    const float v = a.inv[mat];
    alpha = v * v;
    scl = v;
  }
  constexpr bool tall = TALLF;
  // Transposed output of this block: the mirrored tile (GRAM, POLY off the
  // diagonal) or, on the fp32 path, the next step's X^T (UPDATE).
  bool stage_t = false;
  if constexpr (UPD) stage_t = STAGED_T;
  if constexpr (GRAMK || POLYK) stage_t = ti != tj;
  T* __restrict__ Ts = reinterpret_cast<T*>(smem);
  T* __restrict__ C = nullptr;
  T* __restrict__ Clo = nullptr;  // GRAM: the residual of the stored tile, if asked for
  const T* __restrict__ Ain = nullptr;
  const T* __restrict__ Alo = nullptr;  // POLY: a residual plane added to Ain, if given
  float* __restrict__ Xf = nullptr;
  const bf16_t* __restrict__ Xh = nullptr;
  bf16_t* __restrict__ Xh_next = nullptr;
  unsigned char* __restrict__ Xl = nullptr;  // one signed byte per element (lo8_of)
  float* __restrict__ W = nullptr;
  float wscale = 0.f;
  if constexpr (UPD || FINAL) {
    if constexpr (HILO) {
      Xh = static_cast<const bf16_t*>(a.Xh) + (long long)mat * a.sX;
      Xl = static_cast<unsigned char*>(a.Xl) + (long long)mat * a.sX;
      if constexpr (UPD)
        Xh_next = static_cast<bf16_t*>(a.Xh_next) + (long long)mat * a.sX;
    } else {
      Xf = a.Xf + (long long)mat * a.sX;
    }
    if constexpr (FIN_W) {
      W = kernarg<GemmLaunch>().wt.w[mat];
      wscale = a.neg_lr * kernarg<GemmLaunch>().wt.scale[mat];
    }
  } else {
    C = static_cast<T*>(a.C) + (long long)mat * a.sC;
    if constexpr (EPI == EPI_GRAM_LO) Clo = static_cast<T*>(a.Clo) + (long long)mat * a.sC;
    if constexpr (POLYK) Ain = static_cast<const T*>(a.Ain) + (long long)mat * a.sAin;
    if constexpr (EPI == EPI_POLY_LO) Alo = static_cast<const T*>(a.Alo) + (long long)mat * a.sAin;
  }
  const int jl0 = wn * WTN + (lane & 31);

  // FINAL of a tall matrix: the weight (output) is stored transposed to the
  // oriented X, so each lane's 4 consecutive rows i of one column j are
  // contiguous in memory but neighbouring lanes are a row of W apart.  Each
  // 32-row block of every wave goes through LDS instead, as [j][i] rows of
  // 16-byte chunks (chunk c of row j at slot c ^ (j % SCH)), and the block
  // then updates whole 16-byte runs of W's rows, coalesced.  (MIXF: a
  // workgroup-uniform branch on its matrix's orientation.)
  if constexpr (TALLF || MIXF) {
    if (TALLF || ((a.tall_mask >> mat) & 1ull)) {
      constexpr int SR = 32 * WGM;  // staged i per j row
      constexpr int SCH = SR / 4;   // 16-byte chunks per staged row
      constexpr int NCH = BN * SCH;
      constexpr int PERT = NCH / NT;
      static_assert(PERT * NT == NCH, "staged chunks must split over the threads");
      static_assert((size_t)NCH * 16 <= (QROW ? (size_t)STAGE * 16 : LDS_BYTES), "staging fits");
      float* __restrict__ Tf = QROW ? reinterpret_cast<float*>(S0) : reinterpret_cast<float*>(smem);
      // bf16 path: the block's X state (its SR rows, all BN columns) arrives
      // as runs of 8 columns (16 bytes of hi, 8 of lo), coalesced, and waits in
      // the other stage as fp32 rows (columns of rows with bit 2 set XOR 32,
      // so the two half-waves' reads below hit different banks); the next
      // block's runs are loaded during this block's write-back.
      constexpr int RPR = BN / 8;         // runs per X row of the block
      constexpr int RPT = SR * RPR / NT;  // runs per thread and block
      static_assert(!HILO || (QROW && RPT * NT == SR * RPR &&
                              (size_t)SR * BN * 4 <= (size_t)STAGE * 16 && BN % 64 == 0),
                    "the block's X state fits in a stage");
      float* __restrict__ Xs = reinterpret_cast<float*>(S1);
      auto xs_at = [](int il, int jl) __attribute__((always_inline)) {
        return il * BN + (jl ^ (((il >> 2) & 1) << 5));
      };
      [[maybe_unused]] u32x4_t hv[HILO ? RPT : 1];
      [[maybe_unused]] u32x2_t lv[HILO ? RPT : 1];
      auto xload = [&](int mi) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < RPT; ++s) {
          const int u = tid + NT * s, il = u / RPR, jr = u % RPR;
          const long long o =
              (long long)(ti * BM + (il / 32) * WTM + mi * 32 + il % 32) * a.ldx + tj * BN + 8 * jr;
          hv[s] = ldx(reinterpret_cast<const u32x4_t*>(Xh + o));
          lv[s] = ldx(reinterpret_cast<const u32x2_t*>(Xl + o));
        }
      };
      auto xstore = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < RPT; ++s) {
          const int u = tid + NT * s, il = u / RPR, jr = u % RPR;
          float x[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const unsigned hw = hv[s][w], lw = lv[s][w / 2];
            x[2 * w] = lo8_x(__uint_as_float(hw << 16), lo8_byte(lw, 2 * (w % 2)));
            x[2 * w + 1] = lo8_x(__uint_as_float(hw & 0xffff0000u), lo8_byte(lw, 2 * (w % 2) + 1));
          }
          float* d = Xs + xs_at(il, 8 * jr);
          *reinterpret_cast<f32x4_t*>(d) = f32x4_t{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<f32x4_t*>(d + 4) = f32x4_t{x[4], x[5], x[6], x[7]};
        }
      };
      if constexpr (HILO) xload(0);
      static_for<FM>([&](auto mi) {
        if constexpr (HILO) {
          xstore();
          if constexpr (decltype(mi)::value + 1 < FM) xload(decltype(mi)::value + 1);
          __syncthreads();
        }
        [[maybe_unused]] const int ib = i_base + mi * 32 + 4 * hsel;  // + 8q + t
        static_for<FN>([&](auto ni) {
          [[maybe_unused]] const int j = j_base + ni * 32 + (lane & 31);
          const int jl = jl0 + ni * 32;
          float ein[16];
          static_for<16>([&](auto r) {
            if constexpr (HILO) {
              ein[r] = Xs[xs_at(wm * 32 + 8 * (r / 4) + 4 * hsel + r % 4, jl)];
            } else {
              const long long o = (long long)(ib + 8 * (r / 4) + (r % 4)) * a.ldx + j;
              ein[r] = Xf[o];
            }
          });
          static_for<4>([&](auto q) {
            f32x4_t f;
            static_for<4>([&](auto t) {
              constexpr int r = 4 * q + t;
              f[(int)t] = scl * (a.a * ein[r] + acc[mi][ni][r]);
            });
            const int c = (wm * 32 + 8 * q + 4 * hsel) >> 2;
            *reinterpret_cast<f32x4_t*>(Tf + jl * SR + ((c ^ (jl % SCH)) << 2)) = f;
          });
        });
        __syncthreads();
        constexpr int HALF = PERT >= 4 ? 4 : PERT;  // runs per write-back round
        static_assert(PERT % HALF == 0, "write-back rounds");
#pragma unroll
        for (int s0 = 0; s0 < PERT; s0 += HALF) {
          f32x4_t xv[HALF];
          long long off[HALF];
          int nval[HALF];  // valid elements of the run (0 .. 4)
#pragma unroll
          for (int s = 0; s < HALF; ++s) {
            const int cc = tid + NT * (s0 + s), jl = cc / SCH, c = cc % SCH;
            xv[s] = *reinterpret_cast<const f32x4_t*>(Tf + jl * SR + ((c ^ (jl % SCH)) << 2));
            const int il = 4 * c;
            const int i = ti * BM + (il / 32) * WTM + mi * 32 + il % 32;
            const int j = tj * BN + jl;
            const int rem = a.m - i;
            nval[s] = j < a.n ? (rem < 0 ? 0 : rem > 4 ? 4 : rem) : 0;
            off[s] = (long long)j * a.m + i;
          }
          if constexpr (FIN_W) {
            f32x4_t wv[HALF];
#pragma unroll
            for (int s = 0; s < HALF; ++s) {
              if (a.vec_tall && nval[s] == 4) {
                wv[s] = ldx(reinterpret_cast<const f32x4_t*>(W + off[s]));
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) wv[s][t] = t < nval[s] ? W[off[s] + t] : 0.f;
              }
            }
#pragma unroll
            for (int s = 0; s < HALF; ++s) {
              f32x4_t w;
#pragma unroll
              for (int t = 0; t < 4; ++t)
              w[t] = weight_step(wv[s][t], xv[s][t], wscale, a.neg_lrwd, a.cautious);
              if (a.vec_tall && nval[s] == 4) {
                stx(w, reinterpret_cast<f32x4_t*>(W + off[s]));
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (t < nval[s]) W[off[s] + t] = w[t];
              }
            }
          } else {
#pragma unroll
            for (int s = 0; s < HALF; ++s) {
              const long long o = (long long)mat * a.s_out + off[s];
              if (a.out_bf16) {
                bf16_t* ob = static_cast<bf16_t*>(a.out) + o;
                if (a.vec_tall && nval[s] == 4) {
                  uint2 pk;
                  pk.x = (unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(xv[s][0])) |
                         ((unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(xv[s][1])) << 16);
                  pk.y = (unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(xv[s][2])) |
                         ((unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(xv[s][3])) << 16);
                  *reinterpret_cast<uint2*>(ob) = pk;
                } else {
#pragma unroll
                  for (int t = 0; t < 4; ++t)
                    if (t < nval[s]) ob[t] = from_f32<bf16_t>(xv[s][t]);
                }
              } else {
                float* of = static_cast<float*>(a.out) + o;
                if (a.vec_tall && nval[s] == 4) {
                  *reinterpret_cast<f32x4_t*>(of) = xv[s];
                } else {
#pragma unroll
                  for (int t = 0; t < 4; ++t)
                    if (t < nval[s]) of[t] = xv[s][t];
                }
              }
            }
          }
        }
        __syncthreads();  // the staging tile is rewritten by the next block
      });
      return;
    }
  }

  // UPDATE and the FINAL of wide matrices on the bf16 path: X's hi and lo
  // planes move in runs of 8 consecutive columns (16-byte hi and 8-byte lo
  // accesses, 8 lanes per row segment) instead of one element per lane and
  // access, and so do the weights (or the output) where their rows are
  // 16-byte aligned (vec_wide), element by element at ragged edges.  Each wave writes its
  // accumulators of one 32-row block as fp32 rows into its own LDS area and
  // reads them back as runs; the next block's hi and lo are loaded while this
  // one is staged.  Only the wave itself touches its area and a wave's LDS
  // accesses execute in issue order, so a compiler barrier orders them.
  if constexpr ((UPD || (FINAL && !TALLF)) && HILO) {
    constexpr int RPL = WTN / 8;         // runs per staged row
    constexpr int RSTEP = 64 / RPL;      // rows between a lane's runs
    constexpr int RUNS = 32 / RSTEP;     // runs per lane and block
    static_assert(WTN == 64 && RUNS * RSTEP == 32, "64-column wave tiles");
    static_assert(QROW && (size_t)NW * 32 * WTN * 4 <= (size_t)STAGE * 16,
                  "the staged blocks fit in one stage");
    float* __restrict__ Tw = reinterpret_cast<float*>(S0) + wave * 32 * WTN;
    // 16-byte unit u of staged row r sits at unit u ^ (r & 1) ^ 8 ((r >> 2) & 1):
    // the accumulator writes (rows r and r + 4 in the two half-waves) and the
    // run reads (two rows per 16 lanes) are free of bank conflicts
    auto slot = [](int r, int c) __attribute__((always_inline)) {
      return r * WTN + ((((c >> 2) ^ (r & 1) ^ (((r >> 2) & 1) << 3))) << 2) + (c & 3);
    };
    const int rr0 = lane / RPL, cc = 8 * (lane % RPL);  // run s: row rr0 + RSTEP s
    auto offset = [&](int mi, int s) __attribute__((always_inline)) {
      return (long long)(i_base + mi * 32 + rr0 + RSTEP * s) * a.ldx + j_base + cc;
    };
    u32x4_t hv[2][RUNS];
    u32x2_t lv[2][RUNS];
    auto load = [&](auto mi, auto b) __attribute__((always_inline)) {
      static_for<RUNS>([&](auto s) {
        const long long o = offset(decltype(mi)::value, s);
        hv[decltype(b)::value][s] = ldx(reinterpret_cast<const u32x4_t*>(Xh + o));
        lv[decltype(b)::value][s] = ldx(reinterpret_cast<const u32x2_t*>(Xl + o));
      });
    };
    load(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    static_for<FM>([&](auto mi) {
      constexpr int b = decltype(mi)::value & 1;
      if constexpr (decltype(mi)::value + 1 < FM)
        load(std::integral_constant<int, decltype(mi)::value + 1>{},
             std::integral_constant<int, b ^ 1>{});
      static_for<FN>([&](auto ni) {
        static_for<16>([&](auto r) {
          Tw[slot(8 * (r / 4) + 4 * hsel + r % 4, 32 * ni + (lane & 31))] = acc[mi][ni][(int)r];
        });
      });
      asm volatile("" ::: "memory");
      // FINAL: this block's weights (or nothing, for the output), loaded
      // before the block is staged
      [[maybe_unused]] f32x4_t wv[FIN_W ? RUNS : 1][2];
      if constexpr (FIN_W) {
        static_for<RUNS>([&](auto s) {
          const int i = i_base + mi * 32 + rr0 + RSTEP * s, j = j_base + cc;
          const float* Wr = W + (long long)i * a.n + j;
          if (i < a.m && a.vec_wide && j + 8 <= a.n) {
            wv[s][0] = ldx(reinterpret_cast<const f32x4_t*>(Wr));
            wv[s][1] = ldx(reinterpret_cast<const f32x4_t*>(Wr + 4));
          } else {
            static_for<8>([&](auto e) {
              wv[s][e / 4][e % 4] = i < a.m && j + e < a.n ? Wr[(int)e] : 0.f;
            });
          }
        });
      }
      static_for<RUNS>([&](auto s) {
        const int r = rr0 + RSTEP * s;
        const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(Tw + slot(r, cc));
        const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(Tw + slot(r, cc + 4));
        if constexpr (FINAL) {
          float x[8];
          static_for<4>([&](auto w) {
            const unsigned hw = hv[b][s][(int)w], lw = lv[b][s][(int)w / 2];
            static_for<2>([&](auto h) {
              constexpr int e = 2 * w + h;
              const float xe =
                  lo8_x(__uint_as_float(h ? hw & 0xffff0000u : hw << 16), lo8_byte(lw, e % 4));
              x[e] = scl * (a.a * xe + (e < 4 ? p0[e & 3] : p1[e & 3]));
            });
          });
          const int i = i_base + mi * 32 + r, j = j_base + cc;
          if (i < a.m) {
            const bool full = a.vec_wide && j + 8 <= a.n;
            if constexpr (FIN_W) {
              float* Wr = W + (long long)i * a.n + j;
              f32x4_t w0, w1;
              static_for<4>([&](auto t) {
                w0[(int)t] = weight_step(wv[s][0][(int)t], x[t], wscale, a.neg_lrwd, a.cautious);
                w1[(int)t] = weight_step(wv[s][1][(int)t], x[4 + t], wscale, a.neg_lrwd, a.cautious);
              });
              if (full) {
                stx(w0, reinterpret_cast<f32x4_t*>(Wr));
                stx(w1, reinterpret_cast<f32x4_t*>(Wr + 4));
              } else {
                static_for<8>([&](auto e) {
                  if (j + e < a.n) Wr[(int)e] = e < 4 ? w0[e & 3] : w1[e & 3];
                });
              }
            } else {
              const long long oo = (long long)mat * a.s_out + (long long)i * a.n + j;
              if (a.out_bf16) {
                bf16_t* ob = static_cast<bf16_t*>(a.out) + oo;
                if (full) {
                  u32x4_t pk;
                  static_for<4>([&](auto w) {
                    pk[(int)w] =
                        (unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(x[2 * w])) |
                        ((unsigned)__builtin_bit_cast(unsigned short,
                                                      from_f32<bf16_t>(x[2 * w + 1])) << 16);
                  });
                  *reinterpret_cast<u32x4_t*>(ob) = pk;
                } else {
                  static_for<8>([&](auto e) {
                    if (j + e < a.n) ob[(int)e] = from_f32<bf16_t>(x[e]);
                  });
                }
              } else {
                float* of = static_cast<float*>(a.out) + oo;
                if (full) {
                  *reinterpret_cast<f32x4_t*>(of) = f32x4_t{x[0], x[1], x[2], x[3]};
                  *reinterpret_cast<f32x4_t*>(of + 4) = f32x4_t{x[4], x[5], x[6], x[7]};
                } else {
                  static_for<8>([&](auto e) {
                    if (j + e < a.n) of[(int)e] = x[e];
                  });
                }
              }
            }
          }
        } else {
        u32x4_t ho;
        u32x2_t lo = {0u, 0u};
        [[maybe_unused]] float ss = 0.f;
        static_for<4>([&](auto w) {
          const unsigned hw = hv[b][s][(int)w], lw = lv[b][s][(int)w / 2];
          unsigned short hb[2];
          static_for<2>([&](auto h) {
            constexpr int e = 2 * w + h;
            const float x =
                lo8_x(__uint_as_float(h ? hw & 0xffff0000u : hw << 16), lo8_byte(lw, e % 4));
            const float accv = e < 4 ? p0[e & 3] : p1[e & 3];
            const float xn = scl * (a.a * x + accv);
            if constexpr (ROWS) ss = fmaf(xn, xn, ss);
            const bf16_t vh = from_f32<bf16_t>(xn);
            hb[h] = __builtin_bit_cast(unsigned short, vh);
            lo[e / 4] |= lo8_of(xn, to_f32(vh)) << (8 * (e % 4));
          });
          ho[(int)w] = (unsigned)hb[0] | ((unsigned)hb[1] << 16);
        });
        const long long o = offset(mi, s);
        // lo is updated in place: only this block reads X[i][j]'s lo
        stx(ho, reinterpret_cast<u32x4_t*>(Xh_next + o));
        stx(lo, reinterpret_cast<u32x2_t*>(Xl + o));
        if constexpr (ROWS) {
          // the row's sum over the wave's 64 columns, from the 8 lanes of
          // its runs in a fixed butterfly order (all lanes are active here)
          ss += __shfl_xor(ss, 1);
          ss += __shfl_xor(ss, 2);
          ss += __shfl_xor(ss, 4);
          if (lane % RPL == 0)
            a.rowpart[(long long)mat * a.s_rp + (long long)(j_base / WTN) * a.ld_rp + i_base +
                      mi * 32 + rr0 + RSTEP * s] = ss;
        }
        }
      });
      asm volatile("" ::: "memory");  // this block's reads before the next one's writes
    });
    return;
  }

  // Epilogue passes: EPN accumulator column blocks and EPQ of the 4 row
  // quads of one 32-row block at a time (FINAL_W has a third input, so its
  // passes are smaller to keep the loads in flight within the registers).
  constexpr int EPN = FIN_W ? 1 : FN;
  constexpr int EPQ = FIN_W ? 2 : 4;
  constexpr int NPQ = 4 / EPQ;
  static_for<FM * (FN / EPN) * NPQ>([&](auto pass) {
    constexpr int mi = decltype(pass)::value / (FN / EPN * NPQ);
    constexpr int n0 = decltype(pass)::value / NPQ % (FN / EPN) * EPN;
    constexpr int q0 = decltype(pass)::value % NPQ * EPQ;
    const int ib = i_base + mi * 32 + 4 * hsel;  // + 8q + t
    // phase 1: the inputs of this pass
    float ein[EPN][4 * EPQ];
    float win[FIN_W ? EPN : 1][4 * EPQ];
    static_for<EPN>([&](auto nn) {
      const int j = j_base + (n0 + nn) * 32 + (lane & 31);
      static_for<4 * EPQ>([&](auto e) {
        const int i = ib + 8 * (q0 + e / 4) + (e % 4);
        if constexpr (POLYK) ein[nn][e] = to_f32(Ain[(long long)i * a.ldc + j]);
        if constexpr (EPI == EPI_POLY_LO) ein[nn][e] += to_f32(Alo[(long long)i * a.ldc + j]);
        if constexpr (UPD || FINAL) {
          const long long o = (long long)i * a.ldx + j;
          if constexpr (HILO) ein[nn][e] = lo8_x(to_f32(Xh[o]), (int)(signed char)Xl[o]);
          else ein[nn][e] = Xf[o];
        }
        if constexpr (FIN_W) {
          // outside the matrix (zero padding) read element 0 and discard it
          const bool inb = i < a.m && j < a.n;
          const long long oo = tall ? (long long)j * a.m + i : (long long)i * a.n + j;
          win[nn][e] = W[inb ? oo : 0];
        }
      });
    });
    // phase 2: values, direct stores, transposed staging
    static_for<EPN>([&](auto nn) {
      constexpr int ni = n0 + decltype(nn)::value;
      const int j = j_base + ni * 32 + (lane & 31);
      static_for<EPQ>([&](auto qq) {
        constexpr int q = q0 + decltype(qq)::value;
        float v[4];
        static_for<4>([&](auto t) {
          constexpr int r = 4 * q + t;           // accumulator register
          constexpr int e = 4 * decltype(qq)::value + t;  // input of this pass
          const int i = ib + 8 * q + t;
          const float accv = acc[mi][ni][r];
          if constexpr (GRAMK) {
            v[t] = accv * alpha;
            const T hi = from_f32<T>(v[t]);
            C[(long long)i * a.ldc + j] = hi;
            if constexpr (EPI == EPI_GRAM_LO)
              Clo[(long long)i * a.ldc + j] = from_f32<T>(v[t] - to_f32(hi));
          } else if constexpr (POLYK) {
            v[t] = a.b * ein[nn][e] + a.c * accv;
            C[(long long)i * a.ldc + j] = from_f32<T>(v[t]);
          } else if constexpr (UPD) {
            v[t] = scl * (a.a * ein[nn][e] + accv);
            const long long o = (long long)i * a.ldx + j;
            if constexpr (HILO) {
              // lo is updated in place: only this block reads X[i][j]'s lo
              const bf16_t hi = from_f32<bf16_t>(v[t]);
              Xh_next[o] = hi;
              Xl[o] = (unsigned char)lo8_of(v[t], to_f32(hi));
            } else {
              Xf[o] = v[t];
            }
          } else {  // FINAL_W, FINAL_OUT
            const float x = scl * (a.a * ein[nn][e] + accv);
            if (i < a.m && j < a.n) {
              const long long oo = tall ? (long long)j * a.m + i : (long long)i * a.n + j;
              if constexpr (FIN_W) {
                W[oo] = weight_step(win[nn][e], x, wscale, a.neg_lrwd, a.cautious);
              } else if (a.out_bf16) {
                static_cast<bf16_t*>(a.out)[(long long)mat * a.s_out + oo] = from_f32<bf16_t>(x);
              } else {
                static_cast<float*>(a.out)[(long long)mat * a.s_out + oo] = x;
              }
            }
          }
        });
        if constexpr (STAGED_T) {
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
  if constexpr (STAGED_T) {
    if (stage_t) {
      __syncthreads();
      T* __restrict__ dst;
      int ld;
      if constexpr (UPD) {
        dst = static_cast<T*>(a.XTo) + (long long)mat * a.sXT;
        ld = a.ldxt;
      } else {
        dst = C;
        ld = a.ldc;
      }
      constexpr int CPT = BM / EPC;  // 16-byte chunks per transposed row
#pragma unroll 4
      for (int c = tid; c < BN * CPT; c += NT) {
        const int jl = c / CPT, il = (c % CPT) * EPC;
        *reinterpret_cast<u32x4_t*>(dst + (long long)(tj * BN + jl) * ld + ti * BM + il) =
            *reinterpret_cast<const u32x4_t*>(Ts + jl * TLD + il);
      }
    }
  }
}

// bf16: 256x256 tiles on 8 waves (2x4, 128x64 each) or 128x128 tiles on 4
// waves (2x2, 64x64 each), both with the direct-to-LDS main loop; buffer
// loads except for the FINALs, whose epilogue-heavy tiles measured faster
// with global ones (MUON_LOADS=global|buffer overrides, a tuning knob).  The
// bf16 UPDATE / FINAL read X's hi plane as a row-major second operand.
// fp32: 128x128 tiles on 4 waves with register-staged loads.
inline bool buffer_loads(int epi) {
  static const int v = [] {
    const char* e = std::getenv("MUON_LOADS");
    if (!e) return -1;
    return std::strcmp(e, "buffer") == 0 ? 1 : std::strcmp(e, "global") == 0 ? 0 : -1;
  }();
  if (v >= 0) return v == 1;
  return !(epi == EPI_FINAL_W || epi == EPI_FINAL_OUT || epi == EPI_FINAL_W_T ||
           epi == EPI_FINAL_OUT_T || epi == EPI_FINAL_W_MIX);
}

template <typename T, int E>
inline void launch_gemm_t(int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                          hipStream_t s) {
  const GemmLaunch launch{a, t};
  constexpr bool QR = sizeof(T) == 2 && E != EPI_GRAM && E != EPI_POLY && E != EPI_GRAM_LO &&
                     E != EPI_POLY_LO;
  if constexpr (sizeof(T) == 2) {
    // buffer loads address an operand panel with 32-bit lane offsets: up to
    // `tile` rows of the leading dimension
    const long long ld = a.ldp > a.ldq ? a.ldp : a.ldq;
    const bool buf = buffer_loads(E) && (long long)tile * ld * (long long)sizeof(T) < (1LL << 31);
    auto go = [&](auto strm) {
      constexpr bool ST = decltype(strm)::value;
      // the mixed-orientation FINAL exists as 128 x 128 tiles only (with both
      // epilogues in one kernel the 256 x 256 tile runs out of registers)
      if constexpr (E != EPI_FINAL_W_MIX) {
        if (tile == 256) {
          if (buf)
            hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 2, QR, true, ST>), grid,
                               dim3(512), 0, s, launch);
          else
            hipLaunchKernelGGL((gemm_kernel<T, E, 256, 256, 2, 4, 2, QR, false, ST>), grid,
                               dim3(512), 0, s, launch);
          return;
        }
      }
      if (buf)
        hipLaunchKernelGGL((gemm_kernel<T, E, 128, 128, 2, 2, 2, QR, true, ST>), grid,
                           dim3(256), 0, s, launch);
      else
        hipLaunchKernelGGL((gemm_kernel<T, E, 128, 128, 2, 2, 2, QR, false, ST>), grid,
                           dim3(256), 0, s, launch);
    };
    // streaming accesses exist only in the row-major-X (UPDATE / FINAL) epilogues
    if (QR && a.stream)
      go(std::integral_constant<bool, QR>{});
    else
      go(std::false_type{});
    return;
  }
  hipLaunchKernelGGL((gemm_kernel<T, E, 128, 128, 2, 2, 0, QR, false, false>), grid, dim3(256),
                     0, s, launch);
}

// Per-family launchers, one translation unit each (gemm_*.hip).
void launch_gemm_gram(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                      hipStream_t s);
void launch_gemm_poly(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                      hipStream_t s);
void launch_gemm_update(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                        hipStream_t s);
void launch_gemm_final_w(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                         hipStream_t s);
void launch_gemm_final_out(int epi, int tile, const GemmArgs& a, const WeightTable& t, dim3 grid,
                           hipStream_t s);
void launch_gemm_fp32(int epi, const GemmArgs& a, const WeightTable& t, dim3 grid, hipStream_t s);

}  // namespace muon
