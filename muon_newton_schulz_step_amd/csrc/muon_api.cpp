// Host runtime of libmuon.so: argument checks (pure host code, no HIP call,
// so they run on a machine without a GPU), grouping by oriented shape,
// workspace layout, launch sequencing and the optional per-launch timing log.
//
// Sequence per group of same-oriented-shape matrices (the web3.cnoyu.systems
// review of karpathy/autoresearch's train.py, Muon paragraph: momentum,
// Newton-Schulz steps, update), on the caller's stream:
//   prep, norm, then for each step k: gram, poly, update.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "muon.h"
#include "muon_kernels.h"

using namespace muon;

namespace {

constexpr size_t kWsAlign = MUON_WORKSPACE_ALIGN;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
long long pad_dim(long long d) { return (d + kPad - 1) / kPad * kPad; }

bool is_dtype(int d) { return d == MUON_BF16 || d == MUON_FP32; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_finite(float x) { return std::isfinite(x); }

// MUON_GEMM_TILE=128|256 forces the bf16 GEMM tile (a tuning knob).
int tile_pref() {
  static const int v = [] {
    const char* e = std::getenv("MUON_GEMM_TILE");
    return e ? std::atoi(e) : 0;
  }();
  return v;
}

// MUON_GROUP_M=<n> sets the tile rows per scheduling group of full grids.
int group_m() {
  static const int v = [] {
    const char* e = std::getenv("MUON_GROUP_M");
    const int g = e ? std::atoi(e) : 8;
    return g >= 1 ? g : 8;
  }();
  return v;
}

// MUON_STREAM=0|1 forces the cached or the streaming kernel variants for
// every chunk (a testing and tuning knob; see kStreamBytes).
int stream_pref() {
  static const int v = [] {
    const char* e = std::getenv("MUON_STREAM");
    return e ? (std::atoi(e) != 0 ? 1 : 0) : -1;
  }();
  return v;
}

// What a GEMM launch computes, for its choice of tile: every tile of the
// output (update, final), the lower triangle (polynomial, the Q A Q
// products), or the lower triangle of the Gram matrix.
enum class TileUse { full, tri, gram };

// Tile of a bf16 GEMM launch of `batch` matrices with t256 tiles each at
// 256 x 256 (tri, gram: the lower triangle of t256 x t256 tiles, so at
// 128 x 128 the triangle of 2 t256 x 2 t256; full: four times as many).
// A launch runs in rounds over the 256 CUs: a 256-tile workgroup fills a
// CU, two 128-tile workgroups share one.  A round of 128-tile workgroups
// takes about 1/1.6 of a round of 256-tile ones (four times fewer flops
// each, half the operand reuse; 1/1.4 for the Gram, whose epilogue is the
// lightest), so the larger tile wins when 1.6 (1.4) x rounds(256) <=
// rounds(128).  The ratios are fitted to single-chunk steps of 4 to 64
// matrices from 768 x 768 to 2048 x 8192 timed at both tiles.
int pick_tile(bool cbf16, long long t256, int batch, TileUse use) {
  const int pref = tile_pref();
  if (pref == 128 || pref == 256) return gemm_tile(cbf16, pref);
  const bool tri = use != TileUse::full;
  const long long t = tri ? t256 * (t256 + 1) / 2 : t256;
  const long long t128 = tri ? (2 * t256) * (2 * t256 + 1) / 2 : 4 * t256;
  const long long w256 = t * batch, w128 = t128 * batch;
  const long long r256 = (w256 + 255) / 256, r128 = (w128 + 511) / 512;
  const long long ratio5 = use == TileUse::gram ? 7 : 8;  // 5 x the ratio
  return gemm_tile(cbf16, ratio5 * r256 <= 5 * r128 ? 256 : 128);
}

// Workspace regions for `cnt` matrices of oriented shape m x n (padded
// M x N), the X state as described for PrepArgs:
//   bf16: hi plane twice (the update reads one, writes the other), lo plane
//         (one byte per element);
//   fp32: X, X^T twice (read by the update, written by it).
// Then A and B (M x M, compute precision), the norm partials and 1/norm,
// and with NorMuon the per-row scales 1/(sqrt(v') + eps) (M floats) and, on
// the bf16 path, the last update's row sums (N / 64 blocks of M floats).  Groups
// that form some Gram matrices as Q A Q (gram_by_qaq) add A's residual and
// the product T (M x M bf16 each).
struct Layout {
  int m = 0, n = 0, M = 0, N = 0, cnt = 0, nblk = 0;
  bool qaq = false;
  size_t x0 = 0, x1 = 0, x2 = 0, A = 0, B = 0, Alo = 0, T = 0, part = 0, inv = 0, rinv = 0,
         rowpart = 0, total = 0;
  bool rowsums = false;
};

// The Gram matrix of the next step is Q A Q, Q = aI + B (X' = Q X, so
// X' X'^T = Q X X^T Q): two M x M x M products instead of one M x M x N.
// Worth it on the bf16 path when N >= 4M, and only for large M (the two
// launches of small matrices cost more than the one they replace).
bool gram_by_qaq(bool cbf16, long long M, long long N) { return cbf16 && N >= 4 * M && M >= 2048; }

// Steps whose Gram matrix is formed as Q A Q: 1 and 3, never the last one.
// Steps 0 and 2 recompute it from X, so the rounding of A does not compound
// over more than one step.
bool qaq_step(int k, int n_steps) { return (k == 1 || k == 3) && k <= n_steps - 2; }

// When the X state resident at one time (the chunk's own, or the sum over
// the chunks of a step that runs them concurrently) is larger than the
// chip's 256 MB last-level cache, the chunks stream it: the UPDATE / FINAL
// epilogues and prep load and store the X state, weights, gradient and
// momentum nontemporally, which leaves L2 to the GEMM operand panels.
// Smaller ones keep X cached for the next launch.  (The d768 GPT set, two
// concurrent chunks of 94 and 189 MB: 1.67 ms cached, 1.57 ms streamed,
// measured with a 2-byte lo plane, when they held 113 and 226 MB.)
constexpr double kStreamBytes = 256.0 * (1 << 20);

// X-state bytes of a chunk of `cnt` matrices of oriented shape m x n:
// bf16 hi twice + the one-byte lo, fp32 X + X^T twice.
double x_state_bytes(int cnt, int m, int n, bool cbf16) {
  return (double)cnt * (double)pad_dim(m) * (double)pad_dim(n) * (cbf16 ? 5.0 : 12.0);
}

bool make_layout(int cnt, int m, int n, bool cbf16, Layout& L, bool normuon = false) {
  const long long M = pad_dim(m), N = pad_dim(n);
  if (M * N > MUON_MAX_ELEMENTS) return false;
  L.m = m; L.n = n; L.M = (int)M; L.N = (int)N; L.cnt = cnt;
  L.nblk = (int)((M / kPrepTile) * (N / kPrepTile));
  const size_t es = cbf16 ? 2 : 4;
  const size_t MN = (size_t)M * (size_t)N, MM = (size_t)M * (size_t)M;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kWsAlign);
    return o;
  };
  L.x0 = take((size_t)cnt * MN * es);  // bf16: hi 0   fp32: X
  L.x1 = take((size_t)cnt * MN * es);  // bf16: hi 1   fp32: X^T 0
  L.x2 = take((size_t)cnt * MN * (cbf16 ? 1 : 4));  // bf16: lo (1 byte)  fp32: X^T 1
  L.A = take((size_t)cnt * MM * es);
  L.B = take((size_t)cnt * MM * es);
  L.qaq = gram_by_qaq(cbf16, M, N);
  if (L.qaq) {
    L.Alo = take((size_t)cnt * MM * es);
    L.T = take((size_t)cnt * MM * es);
  }
  L.part = take((size_t)cnt * (size_t)L.nblk * 4);
  L.inv = take((size_t)cnt * 4);
  if (normuon) L.rinv = take((size_t)cnt * (size_t)M * 4);
  L.rowsums = normuon && cbf16;
  if (L.rowsums) L.rowpart = take((size_t)cnt * (size_t)(N / 64) * (size_t)M * 4);
  L.total = off;
  return true;
}

struct Group {
  int m, n;
  std::vector<int> idx;
};

void plan(int n, const int* rows, const int* cols, std::vector<Group>& groups,
          std::vector<int>* group_of) {
  groups.clear();
  if (group_of) group_of->assign(n, -1);
  for (int i = 0; i < n; ++i) {
    const int m = rows[i] < cols[i] ? rows[i] : cols[i];
    const int nn = rows[i] < cols[i] ? cols[i] : rows[i];
    int g = -1;
    for (size_t k = 0; k < groups.size(); ++k)
      if (groups[k].m == m && groups[k].n == nn) { g = (int)k; break; }
    if (g < 0) {
      groups.push_back(Group{m, nn, {}});
      g = (int)groups.size() - 1;
    }
    groups[g].idx.push_back(i);
    if (group_of) (*group_of)[i] = g;
  }
}

// ------------------------------------------------------------ timing log
std::atomic<int> g_timing{0};
std::mutex g_log_mu;
struct Pending {
  muon_timing_record rec;
  hipEvent_t e0, e1;
};
std::vector<Pending> g_log;

template <class F>
hipError_t timed(int kind, int m, int n, int batch, int step, double flops, double exec_flops,
                 double bytes, hipStream_t s, F&& launch) {
  if (!g_timing.load(std::memory_order_relaxed)) return launch();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  if (err == hipSuccess) err = hipEventRecord(e0, s);
  if (err != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return err;
  }
  err = launch();
  const hipError_t err2 = hipEventRecord(e1, s);
  if (err == hipSuccess) err = err2;
  muon_timing_record r{kind, m, n, batch, step, 0.f, flops, bytes, exec_flops};
  std::lock_guard<std::mutex> lk(g_log_mu);
  g_log.push_back(Pending{r, e0, e1});
  return err;
}

// ------------------------------------------------------------ one chunk
struct Chunk {
  int cnt;
  unsigned long long tall_mask;       // bit q: matrix q of the chunk is tall
  bool momentum;
  int in_bf16;
  const void* in; long long s_in;     // orthogonalize input
  PrepTable pt;                       // step: gradient / momentum pointers
  float mu;
  int final_mode;
  void* out; long long s_out; int out_bf16;
  WeightTable wt;
  float neg_lr;
  float neg_lrwd;                     // -lr * weight decay (0: none)
  int cautious;
  int normuon;                        // NorMuon after the last step
  float beta2, eps2;
  RowTable vt;                        // NorMuon second moments
};

// resident_x: the X-state bytes resident while this chunk runs (its own, or
// those of every chunk running concurrently with it).
int run_chunk(const Chunk& c, const Layout& L, char* ws, const muon_coeff* coeffs, int n_steps,
              float eps, bool cbf16, double resident_x, hipStream_t s) {
  const size_t es = cbf16 ? 2 : 4;
  const long long MN = (long long)L.M * L.N, MM = (long long)L.M * L.M;
  // bf16: Xh[2] (hi planes), Xl; fp32: Xf, XT[2]
  void* Xh[2] = {ws + L.x0, ws + L.x1};
  void* Xl = ws + L.x2;
  float* Xf = reinterpret_cast<float*>(ws + L.x0);
  void* XT[2] = {ws + L.x1, ws + L.x2};
  void* A = ws + L.A;
  void* B = ws + L.B;
  void* Alo = ws + L.Alo;
  void* Tq = ws + L.T;
  float* part = reinterpret_cast<float*>(ws + L.part);
  float* inv = reinterpret_cast<float*>(ws + L.inv);
  const double m = L.m, n = L.n, cnt = c.cnt;
  const double elems = m * n * cnt;
  const double pmn = cnt * (double)MN, pmm = cnt * (double)MM;  // padded elements

  const bool stream = stream_pref() >= 0 ? stream_pref() == 1 : resident_x > kStreamBytes;
  PrepArgs pa{};
  pa.m = L.m; pa.n = L.n; pa.M = L.M; pa.N = L.N;
  pa.stream = stream;
  pa.tall_mask = c.tall_mask;
  pa.tiles_n = L.N / kPrepTile;
  pa.in = c.in; pa.s_in = c.s_in;
  pa.mu = c.mu;
  pa.sX = MN;
  if (cbf16) {
    pa.Xh = Xh[0]; pa.Xl = Xl;
  } else {
    pa.Xf = Xf; pa.XT = XT[0]; pa.sXT = MN;
  }
  pa.partials = part; pa.nblk = L.nblk;
  // reads g (and momentum r/w); writes X_0: hi + lo (3 bytes), or X + X^T
  const double gsz = c.in_bf16 ? 2 : 4;
  const double prep_bytes = elems * (gsz + (c.momentum ? 8.0 : 0.0)) + pmn * (cbf16 ? 3.0 : 8.0);
  hipError_t err = timed(MUON_K_PREP, L.m, L.n, c.cnt, -1, 0.0, 0.0, prep_bytes, s, [&] {
    return launch_prep(c.in_bf16, cbf16, c.momentum, pa, c.pt, c.cnt, s);
  });
  if (err != hipSuccess) return MUON_ERR_HIP;
  err = timed(MUON_K_NORM, L.m, L.n, c.cnt, -1, 0.0, 0.0, cnt * L.nblk * 4.0 + cnt * 4.0, s,
              [&] { return launch_norm(part, L.nblk, eps, inv, c.cnt, s); });
  if (err != hipSuccess) return MUON_ERR_HIP;

  const int t256 = L.M / 256;
  const int tile_gram = pick_tile(cbf16, t256, c.cnt, TileUse::gram);
  const int tile_sym = pick_tile(cbf16, t256, c.cnt, TileUse::tri);
  const int tile_upd = pick_tile(cbf16, (long long)t256 * (L.N / 256), c.cnt, TileUse::full);
  // flops the MFMAs execute: lower-triangle tiles of M x M for the Gram and
  // polynomial launches (K = N or M), all M x N for the update
  auto tri_el = [&](int tile) {
    const double t = L.M / tile;
    return t * (t + 1) / 2 * (double)tile * tile;
  };
  const double x_gram = 2.0 * tri_el(tile_gram) * L.N * cnt,
               x_sym = 2.0 * tri_el(tile_sym) * L.M * cnt;
  const double x_upd = 2.0 * (double)L.M * L.N * L.M;  // per matrix
  for (int k = 0; k < n_steps; ++k) {
    const bool first = k == 0, last = k == n_steps - 1;
    const int cur = k & 1;
    GemmArgs g{};
    g.stream = stream;
    g.inv = first ? inv : nullptr;
    g.a = coeffs[k].a; g.b = coeffs[k].b; g.c = coeffs[k].c;
    g.m = L.m; g.n = L.n; g.tall_mask = c.tall_mask;
    // the Gram and polynomial launches: lower-triangle tiles of M x M
    g.tiles_m = g.tiles_n = L.M / tile_sym; g.tri = 1;

    if (L.qaq && qaq_step(k, n_steps)) {
      // A = Q A Q with the previous step's A (hi + residual) and B,
      // Q = a_{k-1} I + B: T = a A + B A, then A = a T + T B.  Both products
      // are symmetric (Q and A commute), so the POLY kernel forms them from
      // their lower-triangle tiles; B and A, T are symmetric, so B^T = B and
      // A^T = A as its second operand.  Counted as the Gram's flops, half
      // per launch.
      GemmArgs q = g;
      q.inv = nullptr;
      q.b = coeffs[k - 1].a; q.c = 1.f;
      q.K = L.M; q.sP = q.sQ = MM; q.ldp = q.ldq = L.M;
      q.sC = MM; q.ldc = L.M; q.sAin = MM;
      q.P = B; q.Q = A; q.Ain = A; q.Alo = Alo; q.C = Tq;
      err = timed(MUON_K_GRAMQ, L.m, L.n, c.cnt, k, cnt * m * m * n, x_sym, 5.0 * pmm * es, s,
                  [&] { return launch_gemm(cbf16, EPI_POLY_LO, tile_sym, q, c.wt, c.cnt, s); });
      if (err != hipSuccess) return MUON_ERR_HIP;
      q.P = Tq; q.Q = B; q.Ain = Tq; q.Alo = nullptr; q.C = A;
      err = timed(MUON_K_GRAMQ, L.m, L.n, c.cnt, k, cnt * m * m * n, x_sym, 4.0 * pmm * es, s,
                  [&] { return launch_gemm(cbf16, EPI_POLY, tile_sym, q, c.wt, c.cnt, s); });
      if (err != hipSuccess) return MUON_ERR_HIP;
    } else {
      // A = X X^T (K = N); bf16 reads the hi plane.  Before a step whose
      // Gram matrix is Q A Q, A's residual is kept as well.
      g.P = cbf16 ? Xh[cur] : static_cast<void*>(Xf);
      g.Q = g.P;
      g.sP = g.sQ = MN; g.ldp = g.ldq = L.N; g.K = L.N;
      g.C = A; g.sC = MM; g.ldc = L.M;
      g.Clo = L.qaq && qaq_step(k + 1, n_steps) ? Alo : nullptr;
      g.tiles_m = g.tiles_n = L.M / tile_gram;
      err = timed(MUON_K_GRAM, L.m, L.n, c.cnt, k, cnt * 2.0 * m * m * n, x_gram,
                  pmn * es + pmm * es * (g.Clo ? 1.5 : 1.0), s,
                  [&] {
                    return launch_gemm(cbf16, g.Clo ? EPI_GRAM_LO : EPI_GRAM, tile_gram, g, c.wt,
                                       c.cnt, s);
                  });
      if (err != hipSuccess) return MUON_ERR_HIP;
      g.Clo = nullptr;
      g.tiles_m = g.tiles_n = L.M / tile_sym;
    }

    // B = b A + c A A (K = M)
    g.inv = nullptr;
    g.P = g.Q = A; g.sP = g.sQ = MM; g.ldp = g.ldq = L.M; g.K = L.M;
    g.C = B; g.sC = MM; g.ldc = L.M;
    g.Ain = A; g.sAin = MM;
    err = timed(MUON_K_POLY, L.m, L.n, c.cnt, k, cnt * 2.0 * m * m * m, x_sym, 3.0 * pmm * es, s,
                [&] { return launch_gemm(cbf16, EPI_POLY, tile_sym, g, c.wt, c.cnt, s); });
    if (err != hipSuccess) return MUON_ERR_HIP;

    // X <- a X + B X (K = M).  bf16: Q = the hi plane itself, row-major
    // [k][j]; fp32: Q = X^T.
    g.inv = first ? inv : nullptr;
    g.P = B; g.sP = MM; g.ldp = L.M;
    g.K = L.M;
    g.sX = MN; g.ldx = L.N;
    if (cbf16) {
      g.Q = Xh[cur]; g.sQ = MN; g.ldq = L.N;
      g.Xh = Xh[cur]; g.Xh_next = Xh[cur ^ 1]; g.Xl = Xl;
    } else {
      g.Q = XT[cur]; g.sQ = MN; g.ldq = L.M;
      g.Xf = Xf;
      g.XTo = XT[cur ^ 1]; g.sXT = MN; g.ldxt = L.M;
    }
    g.tri = 0; g.tiles_m = L.M / tile_upd; g.tiles_n = L.N / tile_upd;
    g.final_mode = last ? c.final_mode : FINAL_NONE;
    g.group_m = group_m();
    g.out = c.out; g.s_out = c.s_out; g.out_bf16 = c.out_bf16;
    g.neg_lr = c.neg_lr;
    // tall matrices: runs of 4 elements of a stored row (length m) are
    // aligned when m and the output's matrix stride are multiples of 4
    g.vec_tall = L.m % 4 == 0 && (c.final_mode != FINAL_OUT || c.s_out % 4 == 0);
    // wide matrices: runs of 8 elements of a stored row (length n) are
    // 16-byte aligned when n (bf16 output: and the matrix stride) allows
    g.vec_wide = c.final_mode == FINAL_OUT && c.out_bf16
                     ? L.n % 8 == 0 && c.s_out % 8 == 0
                     : L.n % 4 == 0 && (c.final_mode != FINAL_OUT || c.s_out % 4 == 0);
    g.neg_lrwd = c.neg_lrwd;
    g.cautious = c.cautious;
    // reads B and the operand X; the epilogue reads X (bf16: hi + lo, fp32:
    // X) and writes the next X (bf16: hi + lo, fp32: X + X^T), or, on the
    // last step, reads and writes the weights or writes the output
    if (!last || c.normuon) {
      // (with NorMuon the last step is a plain update too, on the bf16 path
      // with the row sums of the result; the weights follow in their own
      // passes below)
      const bool rows = last && L.rowsums;
      if (rows) {
        g.rowpart = reinterpret_cast<float*>(ws + L.rowpart);
        g.ld_rp = L.M;
        g.s_rp = (long long)(L.N / 64) * L.M;
      }
      const double upd_bytes = pmm * es + pmn * es + pmn * (cbf16 ? 3.0 : 4.0) +
                               pmn * (cbf16 ? 3.0 : 8.0) + (rows ? pmn / 16.0 : 0.0);
      err = timed(MUON_K_UPDATE, L.m, L.n, c.cnt, k, cnt * 2.0 * m * m * n, cnt * x_upd, upd_bytes,
                  s, [&] {
        return launch_gemm(cbf16, rows ? EPI_UPDATE_ROWS : EPI_UPDATE, tile_upd, g, c.wt, c.cnt, s);
      });
    } else {
      // The chunk holds its wide matrices first, then the tall ones, which
      // store the result transposed; each part has its own launch, its tile
      // size chosen for its own count.  When both parts are too small for
      // 256 x 256 tiles, the bf16 weight update takes them in one launch of
      // 128 x 128 tiles instead (the kernel branches per matrix), so that
      // they share their rounds of tiles.
      const int ntall = __builtin_popcountll(c.tall_mask);
      const int nwide = c.cnt - ntall;
      const long long t256_mat = (long long)t256 * (L.N / 256);
      const bool mix = cbf16 && c.final_mode == FINAL_WEIGHTS && nwide > 0 && ntall > 0 &&
                       pick_tile(cbf16, t256_mat, nwide > ntall ? nwide : ntall,
                                 TileUse::full) == 128;
      for (int part = 0; part < (mix ? 1 : 2) && err == hipSuccess; ++part) {
        const int b = mix ? c.cnt : part == 0 ? nwide : ntall;
        if (b == 0) continue;
        GemmArgs gf = g;
        gf.mat0 = part == 0 ? 0 : nwide;
        const int tile_f = mix ? 128 : pick_tile(cbf16, t256_mat, b, TileUse::full);
        gf.tiles_m = L.M / tile_f; gf.tiles_n = L.N / tile_f;
        const int epi = mix ? EPI_FINAL_W_MIX
                        : c.final_mode == FINAL_WEIGHTS ? (part ? EPI_FINAL_W_T : EPI_FINAL_W)
                                                        : (part ? EPI_FINAL_OUT_T : EPI_FINAL_OUT);
        const double bm = b, pmn_b = bm * (double)MN, el_b = m * n * bm;
        const double fin_bytes = bm * (double)MM * es + pmn_b * es + pmn_b * (cbf16 ? 3.0 : 4.0) +
                                 (c.final_mode == FINAL_WEIGHTS ? el_b * 8.0
                                                                : el_b * (c.out_bf16 ? 2.0 : 4.0));
        err = timed(MUON_K_FINAL, L.m, L.n, b, k, bm * 2.0 * m * m * n, bm * x_upd, fin_bytes, s,
                    [&] { return launch_gemm(cbf16, epi, tile_f, gf, c.wt, b, s); });
      }
    }
    if (err != hipSuccess) return MUON_ERR_HIP;
  }
  if (c.normuon) {
    // O is the X state after the last step: hi plane n_steps % 2 (+ lo), or
    // the fp32 X.  Row statistics and scales, then the weights.
    float* rinv = reinterpret_cast<float*>(ws + L.rinv);
    NormuonArgs na{};
    na.m = L.m; na.n = L.n; na.M = L.M; na.N = L.N;
    na.sX = MN; na.ldx = L.N;
    na.Xh = Xh[n_steps & 1]; na.Xl = Xl; na.Xf = Xf;
    if (L.rowsums) {
      na.rowpart = reinterpret_cast<const float*>(ws + L.rowpart);
      na.ld_rp = L.M;
      na.s_rp = (long long)(L.N / 64) * L.M;
    }
    na.beta2 = c.beta2; na.eps2 = c.eps2;
    na.rinv = rinv;
    const double rows_read = L.rowsums ? pmn / 16.0 : pmn * 4.0;
    err = timed(MUON_K_NORMUON, L.m, L.n, c.cnt, -1, 0.0, 0.0, rows_read + cnt * L.m * 8.0, s,
                [&] { return launch_normuon_rows(cbf16, na, c.vt, c.cnt, s); });
    if (err != hipSuccess) return MUON_ERR_HIP;
    ApplyArgs aa{};
    aa.m = L.m; aa.n = L.n; aa.M = L.M; aa.N = L.N;
    aa.tall_mask = c.tall_mask;
    aa.tiles_n = L.N / kPrepTile;
    aa.sX = MN; aa.ldx = L.N;
    aa.Xh = Xh[n_steps & 1]; aa.Xl = Xl; aa.Xf = Xf;
    aa.rinv = rinv;
    aa.neg_lr = c.neg_lr; aa.neg_lrwd = c.neg_lrwd; aa.cautious = c.cautious;
    err = timed(MUON_K_APPLY, L.m, L.n, c.cnt, -1, 0.0, 0.0, elems * (cbf16 ? 11.0 : 12.0), s,
                [&] { return launch_apply(cbf16, aa, c.wt, c.cnt, s); });
    if (err != hipSuccess) return MUON_ERR_HIP;
  }
  return MUON_OK;
}

int check_coeffs(const muon_coeff* coeffs, int n_steps, float eps) {
  if (!coeffs || n_steps < 1 || n_steps > MUON_MAX_STEPS) return MUON_ERR_INVALID_ARG;
  for (int k = 0; k < n_steps; ++k)
    if (!is_finite(coeffs[k].a) || !is_finite(coeffs[k].b) || !is_finite(coeffs[k].c))
      return MUON_ERR_INVALID_ARG;
  if (!is_finite(eps) || eps < 0.f) return MUON_ERR_INVALID_ARG;
  return MUON_OK;
}

bool shape_ok(int rows, int cols) {
  if (rows < 1 || cols < 1) return false;
  return pad_dim(rows) * pad_dim(cols) <= MUON_MAX_ELEMENTS;
}

bool overlap(const void* p, size_t pb, const void* q, size_t qb) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + qb && b < a + pb;
}

// Byte ranges of a step's buffers.  True when any two written ranges
// overlap, or a read range overlaps a written one (reads may share memory
// with each other).  Sorting keeps it O(n log n) for large steps.
struct Span {
  uintptr_t lo, hi;
};
bool spans_conflict(std::vector<Span>& written, const std::vector<Span>& read) {
  std::sort(written.begin(), written.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < written.size(); ++i)
    if (written[i].lo < written[i - 1].hi) return true;
  for (const Span& r : read) {
    // the first written range that ends after r starts
    auto it = std::upper_bound(written.begin(), written.end(), r.lo,
                               [](uintptr_t v, const Span& w) { return v < w.hi; });
    if (it != written.end() && it->lo < r.hi) return true;
  }
  return false;
}

// A step's chunks in launch order: each oriented-shape group split into
// chunks of at most kChunk matrices.
struct ChunkRef {
  int g, b0, cnt;
};

void list_chunks(const std::vector<Group>& groups, std::vector<ChunkRef>& out) {
  out.clear();
  for (int g = 0; g < (int)groups.size(); ++g) {
    const int total = (int)groups[g].idx.size();
    for (int b0 = 0; b0 < total; b0 += kChunk)
      out.push_back(ChunkRef{g, b0, total - b0 < kChunk ? total - b0 : kChunk});
  }
}

// MUON_CONCURRENT=0|1 forces the chunks of a step to run one after the
// other or concurrently (a tuning knob; see concurrent_chunks).
int concurrent_pref() {
  static const int v = [] {
    const char* e = std::getenv("MUON_CONCURRENT");
    return e ? (std::atoi(e) != 0 ? 1 : 0) : -1;
  }();
  return v;
}

// A chunk whose update does fewer multiply-adds than this (count x M x N x M,
// padded) is short, and its launches end in partly idle rounds of tiles.  A
// step made only of such chunks runs them concurrently, each on its own
// stream lane and in its own workspace region, so one chunk's tail overlaps
// another's work (d768 GPT set 1.73 -> 1.67 ms, d1280 12.69 -> 12.41 ms);
// larger chunks run one after the other (concurrent large groups evict each
// other's operand panels from L2: the 3.8B set got slower).
constexpr double kConcurrentMacs = 5e11;

bool concurrent_chunks(const std::vector<Group>& groups, const std::vector<ChunkRef>& chunks) {
  if (chunks.size() < 2) return false;
  if (concurrent_pref() >= 0) return concurrent_pref() == 1;
  for (const ChunkRef& c : chunks) {
    const double M = (double)pad_dim(groups[c.g].m), N = (double)pad_dim(groups[c.g].n);
    if (c.cnt * M * N * M >= kConcurrentMacs) return false;
  }
  return true;
}

// Workspace of a step: the largest chunk's layout when chunks run one after
// the other, the sum of them (each chunk in its own region, in chunk order)
// when they run concurrently.  `offsets` (if given) receives each chunk's
// region.  0 for invalid sizes.
size_t step_ws_bytes(int n, const int* rows, const int* cols, int compute, bool normuon,
                     bool allow_concurrent = true, std::vector<size_t>* offsets = nullptr,
                     bool* concurrent = nullptr) {
  if (n < 1 || !rows || !cols || !is_dtype(compute)) return 0;
  for (int i = 0; i < n; ++i)
    if (!shape_ok(rows[i], cols[i])) return 0;
  std::vector<Group> groups;
  plan(n, rows, cols, groups, nullptr);
  std::vector<ChunkRef> chunks;
  list_chunks(groups, chunks);
  const bool conc = allow_concurrent && concurrent_chunks(groups, chunks);
  if (concurrent) *concurrent = conc;
  if (offsets) offsets->clear();
  size_t best = 0, sum = 0;
  for (const ChunkRef& c : chunks) {
    Layout L;
    if (!make_layout(c.cnt, groups[c.g].m, groups[c.g].n, compute == MUON_BF16, L, normuon))
      return 0;
    if (offsets) offsets->push_back(conc ? sum : 0);
    sum += align_up(L.total, kWsAlign);
    if (L.total > best) best = L.total;
  }
  return conc ? sum : best;
}

// Stream lanes for concurrent chunks: per device, kLanes - 1 library streams
// (default priority, non-blocking) beside the caller's, with the events that
// fork them off the caller's stream and join them back (a pattern HIP graph
// capture records as parallel branches).  The per-device mutex keeps one
// call's fork, launches and join together when several host threads step at
// once.
constexpr int kLanes = 4;
constexpr int kMaxDevices = 64;
struct Lanes {
  std::mutex mu;
  bool ready = false;
  hipStream_t s[kLanes - 1];
  hipEvent_t fork, join[kLanes - 1];
};
Lanes g_lanes[kMaxDevices];
std::mutex g_lanes_init;

Lanes* lanes_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_lanes_init);
  Lanes& L = g_lanes[dev];
  if (!L.ready) {
    for (int i = 0; i < kLanes - 1; ++i)
      if (hipStreamCreateWithFlags(&L.s[i], hipStreamNonBlocking) != hipSuccess ||
          hipEventCreateWithFlags(&L.join[i], hipEventDisableTiming) != hipSuccess)
        return nullptr;
    if (hipEventCreateWithFlags(&L.fork, hipEventDisableTiming) != hipSuccess) return nullptr;
    L.ready = true;
  }
  return &L;
}

// The stream lanes of a concurrent step and the allocation-free entry
// point's scratch belong to the calling thread's current device, so a step
// refuses a stream of another device (MUON_ERR_INVALID_ARG, nothing
// enqueued).  A handle the runtime cannot attribute to a device (the null
// stream, special handles) passes; a bad one fails at its first launch.
int check_stream_device(hipStream_t stream) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MUON_ERR_HIP;
  hipDevice_t own = -1;
  if (stream != nullptr && hipStreamGetDevice(stream, &own) == hipSuccess && own != cur)
    return MUON_ERR_INVALID_ARG;
  return MUON_OK;
}

int check_options(const muon_options* o) {
  if (!o) return MUON_OK;
  if (!is_finite(o->weight_decay) || o->weight_decay < 0.f) return MUON_ERR_INVALID_ARG;
  if ((o->cautious != 0 && o->cautious != 1) || (o->normuon != 0 && o->normuon != 1))
    return MUON_ERR_INVALID_ARG;
  if (o->normuon) {
    if (!is_finite(o->beta2) || o->beta2 < 0.f || o->beta2 > 1.f) return MUON_ERR_INVALID_ARG;
    if (!is_finite(o->normuon_eps) || o->normuon_eps < 0.f) return MUON_ERR_INVALID_ARG;
  }
  return MUON_OK;
}

// muon_step and muon_step_ex (opt == nullptr: the plain step).  With a
// workspace source `src` (muon_step_static), the workspace arguments are
// ignored and the source is asked for one once every argument has passed.
int step_impl(int n, const int* rows, const int* cols, void* const* params, int param_dtype,
              const void* const* grads, int grad_dtype, float* const* momentum,
              float* const* second_moment, float mu, float lr, const float* scale,
              const muon_coeff* coeffs, int n_steps, float eps, int compute,
              const muon_options* opt, void* workspace, size_t workspace_bytes,
              hipStream_t stream, const WorkspaceSource* src = nullptr) {
  if (n < 0) return MUON_ERR_INVALID_ARG;
  if (!is_dtype(param_dtype) || !is_dtype(grad_dtype) || !is_dtype(compute))
    return MUON_ERR_INVALID_ARG;
  if (int st = check_coeffs(coeffs, n_steps, eps)) return st;
  if (!is_finite(mu) || !is_finite(lr)) return MUON_ERR_INVALID_ARG;
  if (int st = check_options(opt)) return st;
  const bool normuon = opt && opt->normuon;
  if (n == 0) return MUON_OK;
  if (!rows || !cols || !params || !grads || !momentum || !scale) return MUON_ERR_INVALID_ARG;
  if (normuon && !second_moment) return MUON_ERR_INVALID_ARG;
  const size_t gsz = grad_dtype == MUON_BF16 ? 2 : 4;
  for (int i = 0; i < n; ++i) {
    if (!shape_ok(rows[i], cols[i])) return MUON_ERR_INVALID_ARG;
    if (!params[i] || !grads[i] || !momentum[i]) return MUON_ERR_INVALID_ARG;
    if (!aligned(params[i], MUON_PTR_ALIGN) || !aligned(grads[i], MUON_PTR_ALIGN) ||
        !aligned(momentum[i], MUON_PTR_ALIGN))
      return MUON_ERR_INVALID_ARG;
    if (!is_finite(scale[i])) return MUON_ERR_INVALID_ARG;
    const size_t el = (size_t)rows[i] * cols[i];
    if (overlap(params[i], el * 4, grads[i], el * gsz) ||
        overlap(params[i], el * 4, momentum[i], el * 4) ||
        overlap(grads[i], el * gsz, momentum[i], el * 4))
      return MUON_ERR_INVALID_ARG;
    if (normuon) {
      const void* v = second_moment[i];
      const size_t vb = (size_t)(rows[i] < cols[i] ? rows[i] : cols[i]) * 4;
      if (!v || !aligned(v, 4)) return MUON_ERR_INVALID_ARG;
      if (overlap(v, vb, params[i], el * 4) || overlap(v, vb, grads[i], el * gsz) ||
          overlap(v, vb, momentum[i], el * 4))
        return MUON_ERR_INVALID_ARG;
    }
  }
  {
    // across matrices too: no written buffer may overlap another buffer
    // that is written, nor a gradient
    std::vector<Span> written, read;
    written.reserve(3 * (size_t)n);
    read.reserve(n);
    for (int i = 0; i < n; ++i) {
      const size_t el = (size_t)rows[i] * cols[i];
      auto span = [](const void* p, size_t b) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        return Span{a, a + b};
      };
      written.push_back(span(params[i], el * 4));
      written.push_back(span(momentum[i], el * 4));
      if (normuon)
        written.push_back(span(second_moment[i],
                               (size_t)(rows[i] < cols[i] ? rows[i] : cols[i]) * 4));
      read.push_back(span(grads[i], el * gsz));
    }
    if (spans_conflict(written, read)) return MUON_ERR_INVALID_ARG;
  }
  if (param_dtype != MUON_FP32) return MUON_ERR_UNSUPPORTED;
  // the allocation-free entry point never forks: its scratch holds one chunk
  std::vector<size_t> ws_off;
  bool conc = false;
  const size_t need = step_ws_bytes(n, rows, cols, compute, normuon, src == nullptr, &ws_off,
                                    &conc);
  if (need == 0) return MUON_ERR_INVALID_ARG;
  if (src) {
    if (int st = src->get(need, &workspace, &workspace_bytes)) return st;
  }
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))
    return MUON_ERR_WORKSPACE;
  for (int i = 0; i < n; ++i) {
    const size_t el = (size_t)rows[i] * cols[i];
    if (overlap(workspace, need, params[i], el * 4) ||
        overlap(workspace, need, grads[i], el * gsz) ||
        overlap(workspace, need, momentum[i], el * 4) ||
        (normuon && overlap(workspace, need, second_moment[i],
                            (size_t)(rows[i] < cols[i] ? rows[i] : cols[i]) * 4)))
      return MUON_ERR_INVALID_ARG;
  }

  if (int st = check_stream_device(stream)) return st;

  const bool cbf16 = compute == MUON_BF16;
  std::vector<Group> groups;
  plan(n, rows, cols, groups, nullptr);
  std::vector<ChunkRef> chunks;
  list_chunks(groups, chunks);
  char* ws = static_cast<char*>(workspace);
  double resident_all = 0.0;
  for (const ChunkRef& r : chunks)
    resident_all += x_state_bytes(r.cnt, groups[r.g].m, groups[r.g].n, cbf16);

  // Concurrent chunks: lane 0 is the caller's stream, the others fork off it
  // and are joined back to it at the end (also after a failed launch, so
  // that a stream capture is never left with unjoined branches).
  hipStream_t lane[kLanes] = {stream};
  int nlanes = 1;
  Lanes* lanes = nullptr;
  std::unique_lock<std::mutex> lane_lock;
  if (conc) {
    lanes = lanes_of_current_device();
    if (!lanes) return MUON_ERR_HIP;
    lane_lock = std::unique_lock<std::mutex>(lanes->mu);
    nlanes = (int)chunks.size() < kLanes ? (int)chunks.size() : kLanes;
    if (hipEventRecord(lanes->fork, stream) != hipSuccess) return MUON_ERR_HIP;
    for (int l = 1; l < nlanes; ++l) {
      lane[l] = lanes->s[l - 1];
      if (hipStreamWaitEvent(lane[l], lanes->fork, 0) != hipSuccess) return MUON_ERR_HIP;
    }
  }
  int status = MUON_OK;
  for (size_t ci = 0; ci < chunks.size() && status == MUON_OK; ++ci) {
    const Group& g = groups[chunks[ci].g];
    const int b0 = chunks[ci].b0, cnt = chunks[ci].cnt;
    // Tall and wide matrices of one oriented shape share the launch: the
    // kernels read each matrix's orientation from the mask.
    Chunk c{};
    // wide matrices first, then the tall ones (the last step launches the
    // two orientations separately, each over a contiguous range)
    int order[kChunk];
    int no = 0;
    for (int pass = 0; pass < 2; ++pass)
      for (int q = 0; q < cnt; ++q) {
        const int i = g.idx[b0 + q];
        if ((rows[i] > cols[i]) == (pass == 1)) order[no++] = i;
      }
    for (int q = 0; q < cnt; ++q) {
      const int i = order[q];
      c.pt.g[q] = grads[i];
      c.pt.buf[q] = momentum[i];
      c.wt.w[q] = static_cast<float*>(params[i]);
      c.wt.scale[q] = scale[i];
      if (normuon) c.vt.v[q] = second_moment[i];
      if (rows[i] > cols[i]) c.tall_mask |= 1ull << q;
    }
    Layout L;
    make_layout(cnt, g.m, g.n, cbf16, L, normuon);
    c.cnt = cnt;
    c.momentum = true;
    c.in_bf16 = grad_dtype == MUON_BF16;
    c.mu = mu;
    c.final_mode = FINAL_WEIGHTS;
    c.neg_lr = -lr;
    if (opt) {
      c.neg_lrwd = -lr * opt->weight_decay;
      c.cautious = opt->cautious;
      c.normuon = opt->normuon;
      c.beta2 = opt->beta2;
      c.eps2 = opt->normuon_eps;
    }
    const double resident = conc ? resident_all : x_state_bytes(cnt, g.m, g.n, cbf16);
    status = run_chunk(c, L, ws + ws_off[ci], coeffs, n_steps, eps, cbf16, resident,
                       lane[ci % nlanes]);
  }
  for (int l = 1; l < nlanes; ++l) {
    if (hipEventRecord(lanes->join[l - 1], lane[l]) != hipSuccess ||
        hipStreamWaitEvent(stream, lanes->join[l - 1], 0) != hipSuccess)
      status = MUON_ERR_HIP;
  }
  return status;
}

}  // namespace

namespace muon {
int step_with_source(int n, const int* rows, const int* cols, void* const* params,
                     int param_dtype, const void* const* grads, int grad_dtype,
                     float* const* momentum, float mu, float lr, const float* scale,
                     const muon_coeff* coeffs, int n_steps, float eps, int compute,
                     const WorkspaceSource& src, hipStream_t stream) {
  return step_impl(n, rows, cols, params, param_dtype, grads, grad_dtype, momentum, nullptr, mu,
                   lr, scale, coeffs, n_steps, eps, compute, nullptr, nullptr, 0, stream, &src);
}
}  // namespace muon

extern "C" {

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "MUON_OK: success";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG: invalid argument";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED: unsupported request";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case MUON_ERR_HIP: return "MUON_ERR_HIP: HIP launch or runtime error";
    default: return "unknown muon status";
  }
}

size_t muon_orthogonalize_workspace_bytes(int batch, int rows, int cols, int compute) {
  if (batch < 1 || !shape_ok(rows, cols) || !is_dtype(compute)) return 0;
  Layout L;
  const int cnt = batch < kChunk ? batch : kChunk;
  const int m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
  if (!make_layout(cnt, m, n, compute == MUON_BF16, L)) return 0;
  return L.total;
}

size_t muon_step_workspace_bytes(int n, const int* rows, const int* cols, int compute) {
  return step_ws_bytes(n, rows, cols, compute, false);
}

size_t muon_step_ex_workspace_bytes(int n, const int* rows, const int* cols, int compute,
                                    const muon_options* options) {
  if (check_options(options) != MUON_OK) return 0;
  return step_ws_bytes(n, rows, cols, compute, options && options->normuon);
}

int muon_plan_groups(int n, const int* rows, const int* cols, int* group_of, int* group_m,
                     int* group_n, int* group_count, int* n_groups) {
  if (n < 0 || !n_groups) return MUON_ERR_INVALID_ARG;
  if (n > 0 && (!rows || !cols || !group_of || !group_m || !group_n || !group_count))
    return MUON_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (rows[i] < 1 || cols[i] < 1) return MUON_ERR_INVALID_ARG;
  std::vector<Group> groups;
  std::vector<int> gof;
  plan(n, rows, cols, groups, &gof);
  for (int i = 0; i < n; ++i) group_of[i] = gof[i];
  for (size_t g = 0; g < groups.size(); ++g) {
    group_m[g] = groups[g].m;
    group_n[g] = groups[g].n;
    group_count[g] = (int)groups[g].idx.size();
  }
  *n_groups = (int)groups.size();
  return MUON_OK;
}

int muon_orthogonalize(const void* in, int in_dtype, void* out, int out_dtype, int batch,
                       int rows, int cols, long long batch_stride, const muon_coeff* coeffs,
                       int n_steps, float eps, int compute, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (batch < 0) return MUON_ERR_INVALID_ARG;
  if (!is_dtype(in_dtype) || !is_dtype(out_dtype) || !is_dtype(compute))
    return MUON_ERR_INVALID_ARG;
  if (int st = check_coeffs(coeffs, n_steps, eps)) return st;
  if (batch == 0) return MUON_OK;
  if (!in || !out) return MUON_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols)) return MUON_ERR_INVALID_ARG;
  if (batch_stride < (long long)rows * cols) return MUON_ERR_INVALID_ARG;
  if (!aligned(in, MUON_PTR_ALIGN) || !aligned(out, MUON_PTR_ALIGN)) return MUON_ERR_INVALID_ARG;
  const size_t need = muon_orthogonalize_workspace_bytes(batch, rows, cols, compute);
  if (need == 0) return MUON_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWsAlign))
    return MUON_ERR_WORKSPACE;
  const size_t isz = in_dtype == MUON_BF16 ? 2 : 4, osz = out_dtype == MUON_BF16 ? 2 : 4;
  const size_t span_in = ((size_t)(batch - 1) * batch_stride + (size_t)rows * cols) * isz;
  const size_t span_out = ((size_t)(batch - 1) * batch_stride + (size_t)rows * cols) * osz;
  // exact aliasing (same pointer, same dtype) is safe: each matrix's output
  // lands where its own input was read, and every chunk reads its inputs
  // before writing; anything else that overlaps is refused
  const bool exact_alias = in == out && in_dtype == out_dtype;
  if (!exact_alias && overlap(in, span_in, out, span_out)) return MUON_ERR_INVALID_ARG;
  if (overlap(workspace, need, in, span_in) || overlap(workspace, need, out, span_out))
    return MUON_ERR_INVALID_ARG;

  const bool cbf16 = compute == MUON_BF16;
  const int m = rows < cols ? rows : cols, n = rows < cols ? cols : rows;
  char* ws = static_cast<char*>(workspace);
  for (int b0 = 0; b0 < batch; b0 += kChunk) {
    const int cnt = batch - b0 < kChunk ? batch - b0 : kChunk;
    Layout L;
    make_layout(cnt, m, n, cbf16, L);
    Chunk c{};
    c.cnt = cnt;
    c.tall_mask = rows > cols ? (cnt == 64 ? ~0ull : ((1ull << cnt) - 1)) : 0ull;
    c.momentum = false;
    c.in_bf16 = in_dtype == MUON_BF16;
    c.in = static_cast<const char*>(in) + (size_t)b0 * batch_stride * isz;
    c.s_in = batch_stride;
    c.final_mode = FINAL_OUT;
    c.out = static_cast<char*>(out) + (size_t)b0 * batch_stride * osz;
    c.s_out = batch_stride;
    c.out_bf16 = out_dtype == MUON_BF16;
    if (int st = run_chunk(c, L, ws, coeffs, n_steps, eps, cbf16,
                           x_state_bytes(cnt, m, n, cbf16), stream))
      return st;
  }
  return MUON_OK;
}

int muon_step(int n, const int* rows, const int* cols, void* const* params, int param_dtype,
              const void* const* grads, int grad_dtype, float* const* momentum, float mu,
              float lr, const float* scale, const muon_coeff* coeffs, int n_steps, float eps,
              int compute, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return step_impl(n, rows, cols, params, param_dtype, grads, grad_dtype, momentum, nullptr, mu,
                   lr, scale, coeffs, n_steps, eps, compute, nullptr, workspace,
                   workspace_bytes, stream);
}

int muon_step_ex(int n, const int* rows, const int* cols, void* const* params, int param_dtype,
                 const void* const* grads, int grad_dtype, float* const* momentum,
                 float* const* second_moment, float mu, float lr, const float* scale,
                 const muon_coeff* coeffs, int n_steps, float eps, int compute,
                 const muon_options* options, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return step_impl(n, rows, cols, params, param_dtype, grads, grad_dtype, momentum,
                   second_moment, mu, lr, scale, coeffs, n_steps, eps, compute, options,
                   workspace, workspace_bytes, stream);
}

int muon_probe_mfma_bf16(int blocks, int iters, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || !sink || !aligned(sink, 4)) return MUON_ERR_INVALID_ARG;
  return launch_mfma_probe(blocks, iters, sink, stream) == hipSuccess ? MUON_OK : MUON_ERR_HIP;
}

int muon_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || blocks < 1 || bytes == 0 || bytes % 16 != 0 || !aligned(src, 16) ||
      !aligned(dst, 16) || overlap(src, bytes, dst, bytes))
    return MUON_ERR_INVALID_ARG;
  return launch_copy_probe(src, dst, (long long)(bytes / 16), blocks, stream) == hipSuccess
             ? MUON_OK
             : MUON_ERR_HIP;
}

int muon_timing_enable(int on) { return g_timing.exchange(on ? 1 : 0); }

int muon_timing_read(muon_timing_record* out, int cap, int* n_out) {
  std::vector<Pending> log;
  {
    std::lock_guard<std::mutex> lk(g_log_mu);
    log.swap(g_log);
  }
  int st = MUON_OK, w = 0;
  for (Pending& p : log) {
    float ms = 0.f;
    if (hipEventSynchronize(p.e1) != hipSuccess || hipEventElapsedTime(&ms, p.e0, p.e1) != hipSuccess)
      st = MUON_ERR_HIP;
    p.rec.ms = ms;
    if (out && w < cap) out[w++] = p.rec;
    (void)hipEventDestroy(p.e0);
    (void)hipEventDestroy(p.e1);
  }
  if (n_out) *n_out = w;
  return st;
}

}  // extern "C"
