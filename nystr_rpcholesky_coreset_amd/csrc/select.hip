// RPNys pivot selection on gfx950: randomly pivoted partial Cholesky of
// H = h_tau(K, K), h_tau(x, y) = exp(beta <x, y> / tau^2), in float64.
//
// [WildCat (arXiv 2602.10056), RPNys / Alg. 1 paragraph.]  Each round draws a
// pivot from the residual diagonal, evaluates the kernel column at the pivot,
// subtracts what the factor already explains, scales by 1/sqrt of the residual
// at the pivot and downdates the residual diagonal.  Only the factor columns,
// the diagonal and n kernel entries per round are touched (O(nr) entries).
//
// GPU structure (units in groups, one streaming launch per round and group,
// see launch_select_t):
//   * workgroup (blk, u) owns 128 consecutive keys of unit u, two per lane;
//     its 4 waves split the previous factor columns j < i (and the key
//     dimensions) into quarters, so every wave streams its own contiguous run
//     of 1 KiB factor segments with 16-byte loads; the partial sums meet in
//     LDS and are combined in a fixed order;
//   * the factor F is stored block-major, [u][blk][j][128]: everything one
//     workgroup ever reads or writes of F is one contiguous region, and a
//     round streams it front to back (one 1 KiB row per column j);
//   * the pivot row F[s, :i] and k_s sit in LDS and are read as broadcasts;
//   * wave 0 finishes the rows: kernel value, new factor column, residual
//     downdate, and a wave-level inclusive prefix sum of the new residuals
//     whose total goes to a per-workgroup slot;
//   * one workgroup per unit, in a later launch, then draws the next pivot
//     with a two-level inverse CDF over those totals and gathers F[s, :i+1]
//     and k_s for the next round (rpc_draw, or extra workgroups of the other
//     group's streaming launch in rpc_fused).  Keeping the draw out of the
//     launch that produced its inputs keeps the streaming kernel free of
//     device-scope fences and atomics (on gfx950 every device-scope release
//     fence writes back the XCD's L2); the kernel boundary publishes the
//     round's results once.
// The draw is in fp64 with a fixed summation order: the prefix C_l of an index
// is (exclusive prefix of its workgroup total) + (in-workgroup inclusive
// prefix), T is C of the last index, and the pivot is the first l with
// C_l > u_i T -- the oracle's rule, up to the rounding of the sums.
#include <climits>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "keymean.hpp"
#include "layout.hpp"

namespace wc {

struct SelectArgs {
  const void* K;        // [U][n][D] fp32 or bf16
  const double* u;      // [U][r]
  int32_t* S;           // [U][r]
  double* L;            // [U][r][r]
  void* F;              // [U][nb][r][RB] block-major factor, float64 or float32 (TF)
  double* dres;         // [U][npad]
  double* bsum;         // [U][nb]
  double* pivbuf;       // [U][2][pbs]
  double* T0;           // [U]
  double* kbar;         // [U][D]
  double* kpart;        // [U][mean_blocks(n)][D] partial key sums (recentring)
  int32_t* stopped;     // [U]
  int32_t* reff;        // [U]
  int n, npad, nb, r, pbs;
  int jkeep;            // columns j < jkeep are read with ordinary loads in every round
  int u0;               // first unit of the launch (unit groups, see launch_select_t)
  double c;             // beta / tau^2
};

constexpr int RB = kSelRowsPerBlock;   // 128 rows per workgroup, 2 per lane of one wave
constexpr double kStopRel = 1e-12;

typedef double d2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

// Two consecutive factor entries as float64: one 16-byte load of float64
// storage, or one 8-byte load of float32 storage converted exactly.
template <typename TF, bool NT>
__device__ __forceinline__ d2v ldf(const TF* p) {
  if constexpr (sizeof(TF) == 8) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const d2v*>(p));
    return *reinterpret_cast<const d2v*>(p);
  } else {
    const f2v v = NT ? __builtin_nontemporal_load(reinterpret_cast<const f2v*>(p)) : *reinterpret_cast<const f2v*>(p);
    return d2v{(double)v.x, (double)v.y};
  }
}

// Key elements as float: chunks of 8 (one 16-byte load for bf16, two for
// fp32) or 4.  Row starts are 16-byte aligned (aligned base, d*elem % 16 == 0).
template <int N> __device__ __forceinline__ void loadk(const bf16_t* p, float (&x)[N]);
template <> __device__ __forceinline__ void loadk<8>(const bf16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}
template <> __device__ __forceinline__ void loadk<4>(const bf16_t* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xFFFF0000u);
  x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
template <int N> __device__ __forceinline__ void loadk(const float* p, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N; q += 4) {
    const float4 a = *reinterpret_cast<const float4*>(p + q);
    x[q] = a.x; x[q + 1] = a.y; x[q + 2] = a.z; x[q + 3] = a.w;
  }
}

// sum_{c in [c0, c0+CN)} (k[c] - kbar[c]) * y[c] in fp64, 4 partial sums.
// SQ: y = k - kbar itself (squared norm).
template <typename TK, int CN, bool RC, bool SQ>
__device__ __forceinline__ double key_part(const TK* krow, int c0, const double* y, const double* kbar) {
  constexpr int CH = CN >= 8 ? 8 : 4;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 2
  for (int c = c0; c < c0 + CN; c += CH) {
    float x[CH];
    loadk<CH>(krow + c, x);
#pragma unroll
    for (int j = 0; j < CH; j += 4) {
      double x0 = x[j], x1 = x[j + 1], x2 = x[j + 2], x3 = x[j + 3];
      if (RC) { x0 -= kbar[c + j]; x1 -= kbar[c + j + 1]; x2 -= kbar[c + j + 2]; x3 -= kbar[c + j + 3]; }
      a0 = fma(x0, SQ ? x0 : y[c + j + 0], a0);
      a1 = fma(x1, SQ ? x1 : y[c + j + 1], a1);
      a2 = fma(x2, SQ ? x2 : y[c + j + 2], a2);
      a3 = fma(x3, SQ ? x3 : y[c + j + 3], a3);
    }
  }
  return (a0 + a1) + (a2 + a3);
}

// In-workgroup inclusive prefix of the 128 residuals, run by one wave (two
// per lane, lane-major).  Owner and selector both use this to get identical
// bits.  Returns the total in every lane.
__device__ __forceinline__ double wave_scan_rows(double (&v)[2]) {
  const int lane = threadIdx.x & (kWave - 1);
  v[1] += v[0];
  const double incl = wave_incl_scan(v[1]);
  double ex = __shfl_up(incl, 1, kWave);
  if (lane == 0) ex = 0.0;
  v[0] = ex + v[0];
  v[1] = ex + v[1];
  return __shfl(v[1], kWave - 1, kWave);
}

__device__ __forceinline__ int wave_min_int(int x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off, kWave));
  return x;
}
__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ void mark_stopped(const SelectArgs& a, int u, int i) {
  if (threadIdx.x == 0) {
    a.stopped[u] = 1;
    a.reff[u] = i;
  }
}

// Prefix of the workgroup totals in rounds of 256 (fixed order).  Calls
// visit(b, P_b, bsum_b) for every block b of the unit, with P_b the exclusive
// prefix, and returns T = P_{nb-1} + bsum_{nb-1} in every thread.
template <typename Visit>
__device__ __forceinline__ double scan_block_totals(const SelectArgs& a, int u, double* scr, Visit visit) {
  const double* bs = a.bsum + (size_t)u * a.nb;
  double carry = 0.0;
  for (int base = 0; base < a.nb; base += kBlock) {
    const int b = base + (int)threadIdx.x;
    const double x = b < a.nb ? bs[b] : 0.0;
    double v[1] = {x}, ex[1], tot;
    block_scan<1>(v, ex, tot, scr);
    const double P = carry + ex[0];
    if (b < a.nb) {
      visit(b, P, x);
      if (b == a.nb - 1) scr[kWavesPerBlock + 1] = P + x;
    }
    carry = carry + tot;
  }
  __syncthreads();
  const double T = scr[kWavesPerBlock + 1];
  __syncthreads();
  return T;
}

// Draw pivot i of unit u and stage it for the launch of round i.  Run by all
// threads of one workgroup after round i-1 (or the initial diagonal).
template <typename TK, int D, bool RC, typename TF>
__device__ void draw_and_stage(const SelectArgs& a, int u, int i, bool is_init, double* smem) {
  double* scr = smem;                              // 16 doubles
  int* iscr = reinterpret_cast<int*>(smem + 16);   // 8 ints
  double* sP = smem + 24;                          // 1 double
  int* sS = reinterpret_cast<int*>(smem + 25);     // 1 int
  double* ks = smem + 32;                          // D doubles
  const int t = threadIdx.x, lane = t & (kWave - 1);

  const double T0pre = is_init ? 0.0 : a.T0[u];
  const double uu = a.u[(size_t)u * a.r + i];
  int myb = INT_MAX, mypos = -1;
  double myP = 0.0, T, target;
  if (a.nb <= kBlock) {
    // One pass: every thread holds at most one workgroup total.
    const int b = t;
    const double x = b < a.nb ? a.bsum[(size_t)u * a.nb + b] : 0.0;
    double v[1] = {x}, ex[1], tot;
    block_scan<1>(v, ex, tot, scr);
    const double P = ex[0];
    if (b == a.nb - 1) scr[kWavesPerBlock + 1] = P + x;
    __syncthreads();
    T = scr[kWavesPerBlock + 1];
    __syncthreads();
    if (is_init && t == 0) a.T0[u] = T;
    const double T0 = is_init ? T : T0pre;
    if (!(T > kStopRel * T0)) { mark_stopped(a, u, i); return; }
    target = uu * T;
    if (b < a.nb) {
      if (P + x > target) { myb = b; myP = P; }
      if (x > 0.0) mypos = b;
    }
  } else {
    // Pass 1: total residual T; pass 2: recompute the same prefixes and find
    // the first block whose last prefix exceeds the target.
    T = scan_block_totals(a, u, scr, [](int, double, double) {});
    if (is_init && t == 0) a.T0[u] = T;
    const double T0 = is_init ? T : T0pre;
    if (!(T > kStopRel * T0)) { mark_stopped(a, u, i); return; }
    target = uu * T;
    scan_block_totals(a, u, scr, [&](int b, double P, double x) {
      if (P + x > target && b < myb) { myb = b; myP = P; }
      if (x > 0.0) mypos = b;
    });
  }
  const int bstar = block_min_int(myb, iscr);
  const bool fallback = (bstar == INT_MAX);
  const int bsel = fallback ? block_max_int(mypos, iscr) : bstar;
  if (bsel < 0) { mark_stopped(a, u, i); return; }   // no mass at all
  if (!fallback && myb == bstar) *sP = myP;
  __syncthreads();
  const double Pb = fallback ? 0.0 : *sP;

  // Rescan the chosen block exactly as its owner did (wave 0): first index
  // with mass whose prefix exceeds the target; the last index with mass in
  // the block if rounding leaves none (and always in the fallback case).
  if (t < kWave) {
    const double* du = a.dres + (size_t)u * a.npad;
    const int row0 = bsel * RB + lane * 2;
    const d2v d0 = *reinterpret_cast<const d2v*>(du + row0);
    double v[2] = {d0.x, d0.y};
    wave_scan_rows(v);
    int cand = INT_MAX, lastpos = -1;
    const double dv[2] = {d0.x, d0.y};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = row0 + k;
      if (l < a.n && dv[k] > 0.0) {
        lastpos = l;
        if (!fallback && Pb + v[k] > target && l < cand) cand = l;
      }
    }
    cand = wave_min_int(cand);
    lastpos = wave_max_int(lastpos);
    if (lane == 0) *sS = cand != INT_MAX ? cand : lastpos;
  }
  __syncthreads();
  const int s = *sS;
  if (s < 0) { mark_stopped(a, u, i); return; }

  // Stage k_s (recentred) and the pivot row F[s, :i]; write row i of L.
  double* pb = a.pivbuf + ((size_t)u * 2 + (i & 1)) * a.pbs;
  const TK* K = reinterpret_cast<const TK*>(a.K) + ((size_t)u * a.n + s) * D;
  for (int c = t; c < D; c += kBlock) {
    double x = (double)Elem<TK>::f32(K, c);
    if (RC) x -= a.kbar[(size_t)u * D + c];
    ks[c] = x;
    pb[2 + a.r + c] = x;
  }
  const TF* Fs = static_cast<const TF*>(a.F) + (((size_t)u * a.nb + s / RB) * a.r) * RB + (s % RB);
  double* Lrow = a.L + ((size_t)u * a.r + i) * a.r;
  double sq = 0.0;
  for (int j = t; j < a.r; j += kBlock) {
    if (j < i) {
      const double f = (double)Fs[(size_t)j * RB];
      pb[2 + j] = f;
      Lrow[j] = f;
      sq = fma(f, f, sq);
    } else if (j > i) {
      Lrow[j] = 0.0;
    }
  }
  __syncthreads();
  double kk = 0.0;
  for (int c = t; c < D; c += kBlock) kk = fma(ks[c], ks[c], kk);
  kk = block_sum(kk, scr);
  sq = block_sum(sq, scr);
  const double gs = exp(a.c * kk) - sq;
  if (!(gs > 0.0)) { mark_stopped(a, u, i); return; }
  if (t == 0) {
    pb[0] = (double)s;
    pb[1] = sqrt(gs);
    a.S[(size_t)u * a.r + i] = s;
  }
}

__global__ __launch_bounds__(kBlock) void rpc_clear(SelectArgs a, int U) {
  const int u = blockIdx.x * kBlock + threadIdx.x;
  if (u < U) {
    a.stopped[u] = 0;
    a.reff[u] = a.r;
  }
}

// Residual diagonal h_tau(k_l, k_l) and its block totals.
template <typename TK, int D, bool RC>
__global__ __launch_bounds__(kBlock) void rpc_init(SelectArgs a) {
  extern __shared__ double smem[];
  double* s_kbar = smem + 32 + D;
  const int u = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
  if (RC) {
    for (int c = t; c < D; c += kBlock) s_kbar[c] = a.kbar[(size_t)u * D + c];
    __syncthreads();
  }
  if (t < kWave) {
    const TK* K = reinterpret_cast<const TK*>(a.K) + (size_t)u * a.n * D;
    double* du = a.dres + (size_t)u * a.npad;
    const int row0 = blk * RB + t * 2;
    double v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = row0 + k;
      v[k] = l < a.n ? exp(a.c * key_part<TK, D, RC, true>(K + (size_t)l * D, 0, nullptr, s_kbar)) : 0.0;
    }
    *reinterpret_cast<d2v*>(du + row0) = d2v{v[0], v[1]};
    const double tot = wave_scan_rows(v);
    if (t == 0) a.bsum[(size_t)u * a.nb + blk] = tot;
  }
}

// Pivot i of every running unit (one workgroup per unit).
template <typename TK, int D, bool RC, typename TF>
__global__ __launch_bounds__(kBlock) void rpc_draw(SelectArgs a, int i) {
  extern __shared__ double smem[];
  const int u = a.u0 + blockIdx.x;
  if (a.stopped[u]) return;
  draw_and_stage<TK, D, RC, TF>(a, u, i, i == 0, smem);
}

// Tuning knobs of the streaming loop (compile-time).
#ifndef WILDCAT_SELECT_CACHED_BYTES
// A round whose factor columns, over all units of the call, total at most this
// many bytes reads them with ordinary loads, so the next round finds them in
// the last-level cache; larger rounds stream them with non-temporal loads.
#define WILDCAT_SELECT_CACHED_BYTES (256ull << 20)
#endif
#ifndef WILDCAT_SELECT_KEEP_BYTES
// In the larger rounds, the keys (read in every round with ordinary loads)
// and the oldest factor columns share this much of the last-level cache: the
// columns that fit beside the keys still take ordinary loads, so every round
// finds them cached.  With the keys at or above it, no column is kept.
#define WILDCAT_SELECT_KEEP_BYTES (224ull << 20)
#endif
#ifndef WILDCAT_SELECT_UNROLL
#define WILDCAT_SELECT_UNROLL 12   // factor loads in flight per lane (8: 171.1 ms, 12: 169.9, 16: 170.6 on the 32k KV-cache workload)
#endif
static_assert(WILDCAT_SELECT_UNROLL % 4 == 0, "the factor loop consumes loads in fours");
#ifndef WILDCAT_SELECT_MINWAVES
#define WILDCAT_SELECT_MINWAVES 1  // minimum waves per SIMD the register budget must allow
#endif

// One RPNys round i for the 128 keys of block blk of unit u.
template <typename TK, int D, bool RC, bool NT, typename TF>
__device__ __forceinline__ void step_block(const SelectArgs& a, int i, int u, int blk, double* smem) {
  double* s_ks = smem + 32;              // D
  double* s_kbar = s_ks + D;             // D
  double* s_pf = s_kbar + D;             // [4][RB] factor partials
  double* s_pk = s_pf + 4 * RB;          // [4][RB] key partials
  double* s_prow = s_pk + 4 * RB;        // r
  const int t = threadIdx.x;
  const int wave = t / kWave, lane = t & (kWave - 1);
  if (a.stopped[u]) return;
  const double* pb = a.pivbuf + ((size_t)u * 2 + (i & 1)) * a.pbs;
  const int s = (int)pb[0];
  const double sgs = pb[1];
  for (int j = t; j < i; j += kBlock) s_prow[j] = pb[2 + j];
  for (int c = t; c < D; c += kBlock) {
    s_ks[c] = pb[2 + a.r + c];
    if (RC) s_kbar[c] = a.kbar[(size_t)u * D + c];
  }
  __syncthreads();

  const int row0 = blk * RB + lane * 2;
  const bool live = row0 < a.n;
  const bool has_y = row0 + 1 < a.n;
  TF* Fb = static_cast<TF*>(a.F) + ((size_t)u * a.nb + blk) * a.r * RB;   // this workgroup's [r][RB] slab
  constexpr size_t ld = RB;

  // This wave's quarter of sum_j F[j][l] F[s][j] for the lane's two rows.
  double fx = 0.0, fy = 0.0;
  if (live) {
    const int jb = (i * wave) >> 2, je = (i * (wave + 1)) >> 2;
    const TF* Fp = Fb + (size_t)jb * ld + 2 * lane;
    double ax0 = 0.0, ay0 = 0.0, ax1 = 0.0, ay1 = 0.0, ax2 = 0.0, ay2 = 0.0, ax3 = 0.0, ay3 = 0.0;
    constexpr int UN = WILDCAT_SELECT_UNROLL;
    int j = jb;
    if (NT) {
      // The oldest columns (j < jkeep over all units of the call fit the
      // last-level cache) take ordinary loads so they stay cached from round
      // to round; whole chunks only, so the accumulation order is unchanged.
      const int jk = a.jkeep < je ? a.jkeep : je;
      const int jm = jk > jb ? jb + (jk - jb) / UN * UN : jb;
      for (; j < jm; j += UN) {
        d2v f[UN];
#pragma unroll
        for (int q = 0; q < UN; ++q) f[q] = ldf<TF, false>(Fp + (size_t)q * ld);
        Fp += UN * ld;
#pragma unroll
        for (int q = 0; q < UN; q += 4) {
          const double p0 = s_prow[j + q], p1 = s_prow[j + q + 1], p2 = s_prow[j + q + 2], p3 = s_prow[j + q + 3];
          ax0 = fma(f[q].x, p0, ax0); ay0 = fma(f[q].y, p0, ay0);
          ax1 = fma(f[q + 1].x, p1, ax1); ay1 = fma(f[q + 1].y, p1, ay1);
          ax2 = fma(f[q + 2].x, p2, ax2); ay2 = fma(f[q + 2].y, p2, ay2);
          ax3 = fma(f[q + 3].x, p3, ax3); ay3 = fma(f[q + 3].y, p3, ay3);
        }
      }
    }
    for (; j + UN <= je; j += UN) {
      d2v f[UN];
#pragma unroll
      for (int q = 0; q < UN; ++q) f[q] = ldf<TF, NT>(Fp + (size_t)q * ld);
      Fp += UN * ld;
#pragma unroll
      for (int q = 0; q < UN; q += 4) {
        const double p0 = s_prow[j + q], p1 = s_prow[j + q + 1], p2 = s_prow[j + q + 2], p3 = s_prow[j + q + 3];
        ax0 = fma(f[q].x, p0, ax0); ay0 = fma(f[q].y, p0, ay0);
        ax1 = fma(f[q + 1].x, p1, ax1); ay1 = fma(f[q + 1].y, p1, ay1);
        ax2 = fma(f[q + 2].x, p2, ax2); ay2 = fma(f[q + 2].y, p2, ay2);
        ax3 = fma(f[q + 3].x, p3, ax3); ay3 = fma(f[q + 3].y, p3, ay3);
      }
    }
    // Remainder: fours, then ones (short rounds spend a large share here).
    for (; j + 4 <= je; j += 4) {
      d2v f[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = ldf<TF, NT>(Fp + (size_t)q * ld);
      Fp += 4 * ld;
      ax0 = fma(f[0].x, s_prow[j], ax0); ay0 = fma(f[0].y, s_prow[j], ay0);
      ax1 = fma(f[1].x, s_prow[j + 1], ax1); ay1 = fma(f[1].y, s_prow[j + 1], ay1);
      ax2 = fma(f[2].x, s_prow[j + 2], ax2); ay2 = fma(f[2].y, s_prow[j + 2], ay2);
      ax3 = fma(f[3].x, s_prow[j + 3], ax3); ay3 = fma(f[3].y, s_prow[j + 3], ay3);
    }
    for (; j < je; ++j) {
      const d2v f0 = ldf<TF, NT>(Fp);
      Fp += ld;
      const double p0 = s_prow[j];
      ax0 = fma(f0.x, p0, ax0); ay0 = fma(f0.y, p0, ay0);
    }
    fx = (ax0 + ax1) + (ax2 + ax3);
    fy = (ay0 + ay1) + (ay2 + ay3);
  }
  // This wave's quarter of <k_l - kbar, k_s - kbar>.
  constexpr int DQ = D / 4;
  double kx = 0.0, ky = 0.0;
  if (live) {
    const TK* K = reinterpret_cast<const TK*>(a.K) + ((size_t)u * a.n + row0) * D;
    kx = key_part<TK, DQ, RC, false>(K, wave * DQ, s_ks, s_kbar);
    if (has_y) ky = key_part<TK, DQ, RC, false>(K + D, wave * DQ, s_ks, s_kbar);
  }
  s_pf[wave * RB + 2 * lane] = fx;
  s_pf[wave * RB + 2 * lane + 1] = fy;
  s_pk[wave * RB + 2 * lane] = kx;
  s_pk[wave * RB + 2 * lane + 1] = ky;
  __syncthreads();

  if (wave == 0) {
    double v[2] = {0.0, 0.0};
    if (live) {
      double* du = a.dres + (size_t)u * a.npad;
      double g[2], fnew[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = 2 * lane + k;
        const double fd = (s_pf[e] + s_pf[RB + e]) + (s_pf[2 * RB + e] + s_pf[3 * RB + e]);
        const double kd = (s_pk[e] + s_pk[RB + e]) + (s_pk[2 * RB + e] + s_pk[3 * RB + e]);
        g[k] = exp(a.c * kd) - fd;
      }
      fnew[0] = g[0] / sgs;
      fnew[1] = has_y ? g[1] / sgs : 0.0;
      if constexpr (sizeof(TF) == 8) {
        *reinterpret_cast<d2v*>(Fb + (size_t)i * ld + 2 * lane) = d2v{fnew[0], fnew[1]};
      } else {
        // float32 storage: round once; the downdate and L use the stored value
        const f2v st = {(float)fnew[0], (float)fnew[1]};
        *reinterpret_cast<f2v*>(Fb + (size_t)i * ld + 2 * lane) = st;
        fnew[0] = (double)st.x;
        fnew[1] = (double)st.y;
      }
      const d2v dold = *reinterpret_cast<const d2v*>(du + row0);
      const double dd[2] = {dold.x, dold.y};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const double f2 = fnew[k] * fnew[k];
        double dn = dd[k] - f2;
        dn = dn > 0.0 ? dn : 0.0;
        if (row0 + k == s) {
          dn = 0.0;
          a.L[((size_t)u * a.r + i) * a.r + i] = fnew[k];
        }
        v[k] = (k == 0 || has_y) ? dn : 0.0;
      }
      *reinterpret_cast<d2v*>(du + row0) = d2v{v[0], v[1]};
    }
    const double tot = wave_scan_rows(v);
    if (lane == 0) a.bsum[(size_t)u * a.nb + blk] = tot;
  }
}

// One RPNys round i for every unit still running.
template <typename TK, int D, bool RC, bool NT, typename TF>
__global__ __launch_bounds__(kBlock, WILDCAT_SELECT_MINWAVES) void rpc_step(SelectArgs a, int i) {
  extern __shared__ double smem[];
  step_block<TK, D, RC, NT, TF>(a, i, a.u0 + blockIdx.y, blockIdx.x, smem);
}

// One launch of the paired schedule: the first ndraw workgroups draw pivot
// di of the units of group `da` (one workgroup per unit), the others run
// round si of group `sa` (nb workgroups per unit).  The two groups are
// disjoint, so the roles touch disjoint data; the draw is the latency-bound
// part and rides along with the other group's streaming.
template <typename TK, int D, bool RC, bool NT, typename TF>
__global__ __launch_bounds__(kBlock, WILDCAT_SELECT_MINWAVES) void rpc_fused(SelectArgs sa, int si, SelectArgs da,
                                                                             int di, int ndraw) {
  extern __shared__ double smem[];
  const int b = blockIdx.x;
  if (b < ndraw) {
    const int u = da.u0 + b;
    if (!da.stopped[u]) draw_and_stage<TK, D, RC, TF>(da, u, di, di == 0, smem);
    return;
  }
  const int k = b - ndraw;
  step_block<TK, D, RC, NT, TF>(sa, si, sa.u0 + k / sa.nb, k % sa.nb, smem);
}

// r_eff, -1 padding of S and zero rows of L past r_eff.
__global__ __launch_bounds__(kBlock) void rpc_finalize(SelectArgs a, int32_t* r_eff_out) {
  const int u = a.u0 + blockIdx.x, t = threadIdx.x;
  const int re = a.stopped[u] ? a.reff[u] : a.r;
  if (t == 0) r_eff_out[u] = re;
  for (int j = re + t; j < a.r; j += kBlock) a.S[(size_t)u * a.r + j] = -1;
  double* Lu = a.L + (size_t)u * a.r * a.r;
  const size_t from = (size_t)re * a.r, to = (size_t)a.r * a.r;
  for (size_t e = from + t; e < to; e += kBlock) Lu[e] = 0.0;
}

// Units are independent, so they are split into contiguous groups whose
// rounds run on separate streams (the caller's stream and auxiliary ones,
// forked and joined with events): while one group draws its next pivot (one
// small workgroup per unit) or drains the tail of its streaming launch,
// other groups' factor streams keep HBM busy.  With an even number of groups
// two groups share a stream and every launch carries one group's round and
// the other group's next draw (rpc_fused), halving the launches per round.
// On the 32k KV-cache workload: select 185.5 ms with one group, 172.3 with
// four groups on four streams, 169.8 with eight groups in pairs on four
// streams.
#ifndef WILDCAT_SELECT_GROUPS
#define WILDCAT_SELECT_GROUPS 8
#endif
#ifndef WILDCAT_SELECT_FUSED
#define WILDCAT_SELECT_FUSED 1      // pairs of groups share a stream, each round's launch carrying the other's draw
#endif
constexpr int kMaxGroups = 8;
constexpr int kMaxDevices = 64;
static_assert(WILDCAT_SELECT_GROUPS >= 1 && WILDCAT_SELECT_GROUPS <= kMaxGroups, "unit groups");

namespace {
// One set of auxiliary streams (default priority, non-blocking) and the
// events that fork them from and join them into the caller's stream.
struct AuxStreams {
  int dev = 0;
  hipStream_t s[kMaxGroups - 1] = {};
  hipEvent_t fork = nullptr, join[kMaxGroups - 1] = {};
};
// Per device, the sets not checked out by a call in progress.  A call takes
// a set for the time it enqueues its work (its own streams and events, so
// concurrent calls from several host threads do not wait for each other) and
// returns it; sets are created when every existing one is taken and kept
// until the process ends.
std::mutex g_aux_mu;
std::vector<AuxStreams*> g_aux_free[kMaxDevices];

hipError_t aux_acquire(AuxStreams** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(g_aux_mu);
    if (!g_aux_free[dev].empty()) {
      *out = g_aux_free[dev].back();
      g_aux_free[dev].pop_back();
      return hipSuccess;
    }
  }
  AuxStreams* x = new AuxStreams;
  x->dev = dev;
  if ((e = hipEventCreateWithFlags(&x->fork, hipEventDisableTiming)) != hipSuccess) return e;
  for (int g = 0; g < kMaxGroups - 1; ++g) {
    if ((e = hipStreamCreateWithFlags(&x->s[g], hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&x->join[g], hipEventDisableTiming)) != hipSuccess) return e;
  }
  *out = x;
  return hipSuccess;
}

// Returns a set to its device's pool (its enqueued work may still be running:
// the next user's launches queue behind it on the same streams).
struct AuxLease {
  AuxStreams* x = nullptr;
  ~AuxLease() {
    if (x == nullptr) return;
    std::lock_guard<std::mutex> lock(g_aux_mu);
    g_aux_free[x->dev].push_back(x);
  }
};
}  // namespace

template <typename TK, int D, bool RC, typename TF>
static hipError_t launch_select_t(const SelectArgs& a, int U, int32_t* r_eff, hipStream_t st) {
  const dim3 grid(a.nb, U);
  rpc_clear<<<(U + kBlock - 1) / kBlock, kBlock, 0, st>>>(a, U);
  if (RC) launch_key_mean<TK, D>(reinterpret_cast<const TK*>(a.K), a.kpart, a.kbar, U, a.n, st);
  const size_t lds_init = (32 + 2 * D) * sizeof(double);
  const size_t lds_draw = (32 + D) * sizeof(double);
  const size_t lds_step = (32 + 2 * D + 8 * RB + a.r) * sizeof(double);
  rpc_init<TK, D, RC><<<grid, kBlock, lds_init, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int G = U < WILDCAT_SELECT_GROUPS ? U : WILDCAT_SELECT_GROUPS;
  const bool paired = WILDCAT_SELECT_FUSED && G >= 2 && G % 2 == 0;
  const int NS = paired ? G / 2 : G;   // streams
  hipStream_t gs[kMaxGroups] = {st};
  SelectArgs ga[kMaxGroups];
  int gU[kMaxGroups];
  AuxLease lease;
  AuxStreams* aux = nullptr;
  if (NS > 1) {
    if ((e = aux_acquire(&aux)) != hipSuccess) return e;
    lease.x = aux;
    if ((e = hipEventRecord(aux->fork, st)) != hipSuccess) return e;
    for (int g = 1; g < NS; ++g) {
      gs[g] = aux->s[g - 1];
      if ((e = hipStreamWaitEvent(gs[g], aux->fork, 0)) != hipSuccess) return e;
    }
  }
  for (int g = 0; g < G; ++g) {
    ga[g] = a;
    ga[g].u0 = (int)((int64_t)U * g / G);
    gU[g] = (int)((int64_t)U * (g + 1) / G) - ga[g].u0;
  }
  const size_t col_bytes = (size_t)U * a.npad * (sizeof(TF));   // one factor column of every unit
  auto cached = [&](int i) { return (size_t)i * col_bytes <= (size_t)WILDCAT_SELECT_CACHED_BYTES; };
  {
    const size_t key_bytes = (size_t)U * a.n * D * sizeof(TK);
    const size_t budget = (size_t)WILDCAT_SELECT_KEEP_BYTES;
    const size_t keep = key_bytes < budget ? (budget - key_bytes) / col_bytes : 0;
    for (int g = 0; g < G; ++g) ga[g].jkeep = (int)(keep < (size_t)a.r ? keep : (size_t)a.r);
  }
  if (paired) {
    // Stream k runs groups A = 2k and B = 2k+1 alternately, each launch one
    // group's round together with the other group's next draw:
    //   [step A_i + draw B_i] [step B_i + draw A_{i+1}] [step A_{i+1} + ...]
    // Every dependency (a draw after its group's previous round, a round
    // after its draw) is on an earlier launch of the same stream.
    for (int k = 0; k < NS; ++k) {
      SelectArgs both = ga[2 * k];   // the pair's units are contiguous
      rpc_draw<TK, D, RC, TF><<<gU[2 * k] + gU[2 * k + 1], kBlock, lds_draw, gs[k]>>>(both, 0);
    }
    for (int i = 0; i < a.r; ++i) {
      for (int k = 0; k < NS; ++k) {
        const int A = 2 * k, B = 2 * k + 1;
        const int nd1 = i >= 1 ? gU[B] : 0;
        const int nd2 = i + 1 < a.r ? gU[A] : 0;
        if (cached(i)) {
          rpc_fused<TK, D, RC, false, TF><<<nd1 + a.nb * gU[A], kBlock, lds_step, gs[k]>>>(ga[A], i, ga[B], i, nd1);
          rpc_fused<TK, D, RC, false, TF><<<nd2 + a.nb * gU[B], kBlock, lds_step, gs[k]>>>(ga[B], i, ga[A], i + 1, nd2);
        } else {
          rpc_fused<TK, D, RC, true, TF><<<nd1 + a.nb * gU[A], kBlock, lds_step, gs[k]>>>(ga[A], i, ga[B], i, nd1);
          rpc_fused<TK, D, RC, true, TF><<<nd2 + a.nb * gU[B], kBlock, lds_step, gs[k]>>>(ga[B], i, ga[A], i + 1, nd2);
        }
      }
    }
    for (int k = 0; k < NS; ++k) {
      SelectArgs both = ga[2 * k];
      rpc_finalize<<<gU[2 * k] + gU[2 * k + 1], kBlock, 0, gs[k]>>>(both, r_eff);
    }
  } else {
    for (int g = 0; g < G; ++g) rpc_draw<TK, D, RC, TF><<<gU[g], kBlock, lds_draw, gs[g]>>>(ga[g], 0);
    for (int i = 0; i < a.r; ++i) {
      for (int g = 0; g < G; ++g) {
        if (cached(i)) rpc_step<TK, D, RC, false, TF><<<dim3(a.nb, gU[g]), kBlock, lds_step, gs[g]>>>(ga[g], i);
        else rpc_step<TK, D, RC, true, TF><<<dim3(a.nb, gU[g]), kBlock, lds_step, gs[g]>>>(ga[g], i);
        if (i + 1 < a.r) rpc_draw<TK, D, RC, TF><<<gU[g], kBlock, lds_draw, gs[g]>>>(ga[g], i + 1);
      }
    }
    for (int g = 0; g < G; ++g) rpc_finalize<<<gU[g], kBlock, 0, gs[g]>>>(ga[g], r_eff);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int g = 1; g < NS; ++g) {
    if ((e = hipEventRecord(aux->join[g - 1], gs[g])) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(st, aux->join[g - 1], 0)) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TK, int D>
static hipError_t launch_select_rc(const SelectArgs& a, int U, bool rc, bool f32, int32_t* r_eff, hipStream_t st) {
  if (f32) return rc ? launch_select_t<TK, D, true, float>(a, U, r_eff, st)
                     : launch_select_t<TK, D, false, float>(a, U, r_eff, st);
  return rc ? launch_select_t<TK, D, true, double>(a, U, r_eff, st)
            : launch_select_t<TK, D, false, double>(a, U, r_eff, st);
}

template <typename TK>
static hipError_t launch_select_d(const SelectArgs& a, int U, int d, bool rc, bool f32, int32_t* r_eff,
                                  hipStream_t st) {
  switch (d) {
    case 16: return launch_select_rc<TK, 16>(a, U, rc, f32, r_eff, st);
    case 32: return launch_select_rc<TK, 32>(a, U, rc, f32, r_eff, st);
    case 64: return launch_select_rc<TK, 64>(a, U, rc, f32, r_eff, st);
    case 128: return launch_select_rc<TK, 128>(a, U, rc, f32, r_eff, st);
  }
  return hipErrorInvalidValue;
}

// Host entry used by the C ABI (arguments already validated).
hipError_t launch_select(int bf16, int U, int n, int d, int r, double c, int recentre, int f32_factor,
                         const void* K, const double* u, int32_t* S, int32_t* r_eff, double* L,
                         void* ws, hipStream_t st) {
  const SelectLayout lay(U, n, d, r, f32_factor ? 4 : 8);
  char* w = static_cast<char*>(ws);
  SelectArgs a;
  a.K = K; a.u = u; a.S = S; a.L = L;
  a.F = w + lay.F;
  a.dres = reinterpret_cast<double*>(w + lay.dres);
  a.bsum = reinterpret_cast<double*>(w + lay.bsum);
  a.pivbuf = reinterpret_cast<double*>(w + lay.pivbuf);
  a.T0 = reinterpret_cast<double*>(w + lay.T0);
  a.kbar = reinterpret_cast<double*>(w + lay.kbar);
  a.kpart = reinterpret_cast<double*>(w + lay.kpart);
  a.stopped = reinterpret_cast<int32_t*>(w + lay.stopped);
  a.reff = reinterpret_cast<int32_t*>(w + lay.reff);
  a.n = n; a.npad = lay.npad; a.nb = lay.nb; a.r = r; a.pbs = lay.pbs; a.u0 = 0; a.jkeep = 0; a.c = c;
  return bf16 ? launch_select_d<bf16_t>(a, U, d, recentre != 0, f32_factor != 0, r_eff, st)
              : launch_select_d<float>(a, U, d, recentre != 0, f32_factor != 0, r_eff, st);
}

}  // namespace wc
