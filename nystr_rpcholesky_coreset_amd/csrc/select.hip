// RPNys pivot selection on gfx950: randomly pivoted partial Cholesky of
// H = h_tau(K, K), h_tau(x, y) = exp(beta <x, y> / tau^2), in float64.
//
// [WildCat (arXiv 2602.10056), RPNys / Alg. 1 paragraph.]  Each round draws a
// pivot from the residual diagonal, evaluates the kernel column at the pivot,
// subtracts what the factor already explains, scales by 1/sqrt of the residual
// at the pivot and downdates the residual diagonal.  Only the factor columns,
// the diagonal and n kernel entries per round are touched (O(nr) entries).
//
// GPU structure (one launch per round, all units in one grid):
//   * workgroup (blk, u) owns 512 consecutive keys of unit u, two per lane;
//     the factor F is stored [u][i][npad] so a round's read of F[:i] streams
//     i contiguous 4 KiB slabs per workgroup with 16-byte loads;
//   * the pivot row F[s, :i] and k_s sit in LDS and are read as broadcasts;
//   * each workgroup writes its slice of the new residual diagonal and a
//     deterministic in-workgroup prefix-sum total; the last workgroup of a unit
//     to finish (device-scope counter) draws the next pivot with a two-level
//     inverse CDF over those totals and gathers F[s, :i+1] and k_s for the
//     next launch, so the next round starts with its pivot ready.
// The draw is in fp64 with a fixed summation order: the prefix C_l of an index
// is (exclusive prefix of its workgroup total) + (in-workgroup inclusive
// prefix), T is C of the last index, and the pivot is the first l with
// C_l > u_i T -- the same rule as the oracle, up to rounding of the sums.
#include <climits>

#include "common.hpp"
#include "layout.hpp"

namespace wc {

struct SelectArgs {
  const void* K;        // [U][n][D] fp32 or bf16
  const double* u;      // [U][r]
  int32_t* S;           // [U][r]
  double* L;            // [U][r][r]
  double* F;            // [U][r][npad]
  double* dres;         // [U][npad]
  double* bsum;         // [U][nb]
  double* pivbuf;       // [U][2][pbs]
  double* T0;           // [U]
  double* kbar;         // [U][D]
  int32_t* stopped;     // [U]
  int32_t* reff;        // [U]
  uint32_t* counter;    // [U]
  int n, npad, nb, r, pbs;
  double c;             // beta / tau^2
};

constexpr int RPT = kSelRowsPerThread;
constexpr int RB = kSelRowsPerBlock;
constexpr double kStopRel = 1e-12;

// Eight consecutive key elements as float (one 16-byte load for bf16, two
// for fp32).  Rows are 16-byte aligned: the C ABI checks the base pointer and
// d*sizeof(elem) is a multiple of 16.
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// <k_l - kbar, ks> in fp64 for one key row; 4 partial sums in a fixed order.
template <typename TK, int D, bool RC>
__device__ __forceinline__ double key_dot(const TK* krow, const double* ks, const double* kbar) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 2
  for (int c = 0; c < D; c += 8) {
    float x[8];
    load8(krow + c, x);
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      double x0 = x[j], x1 = x[j + 1], x2 = x[j + 2], x3 = x[j + 3];
      if (RC) { x0 -= kbar[c + j]; x1 -= kbar[c + j + 1]; x2 -= kbar[c + j + 2]; x3 -= kbar[c + j + 3]; }
      a0 = fma(x0, ks[c + j + 0], a0);
      a1 = fma(x1, ks[c + j + 1], a1);
      a2 = fma(x2, ks[c + j + 2], a2);
      a3 = fma(x3, ks[c + j + 3], a3);
    }
  }
  return (a0 + a1) + (a2 + a3);
}

// ||k_l - kbar||^2 in fp64.
template <typename TK, int D, bool RC>
__device__ __forceinline__ double key_sqnorm(const TK* krow, const double* kbar) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 2
  for (int c = 0; c < D; c += 8) {
    float x[8];
    load8(krow + c, x);
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      double x0 = x[j], x1 = x[j + 1], x2 = x[j + 2], x3 = x[j + 3];
      if (RC) { x0 -= kbar[c + j]; x1 -= kbar[c + j + 1]; x2 -= kbar[c + j + 2]; x3 -= kbar[c + j + 3]; }
      a0 = fma(x0, x0, a0);
      a1 = fma(x1, x1, a1);
      a2 = fma(x2, x2, a2);
      a3 = fma(x3, x3, a3);
    }
  }
  return (a0 + a1) + (a2 + a3);
}

__device__ __forceinline__ void mark_stopped(const SelectArgs& a, int u, int i) {
  if (threadIdx.x == 0) {
    a.stopped[u] = 1;
    a.reff[u] = i;
  }
}

// Prefix of the workgroup totals in rounds of 256 (fixed order).  Calls
// visit(b, P_b, bsum_b) for every block b of the unit, with P_b the exclusive
// prefix, and returns T = P_{nb-1} + bsum_{nb-1}.  Every thread gets T.
template <typename Visit>
__device__ __forceinline__ double scan_block_totals(const SelectArgs& a, int u, double* scr, Visit visit) {
  const double* bs = a.bsum + (size_t)u * a.nb;
  double carry = 0.0, T = 0.0;
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
  T = scr[kWavesPerBlock + 1];
  __syncthreads();
  return T;
}

// Draw pivot i of unit u and stage it for the launch of round i.  Run by all
// threads of the unit's last workgroup of round i-1 (or of the init kernel).
template <typename TK, int D, bool RC>
__device__ void draw_and_stage(const SelectArgs& a, int u, int i, bool is_init, double* smem) {
  double* scr = smem;                              // 16 doubles
  int* iscr = reinterpret_cast<int*>(smem + 16);   // 8 ints
  double* sP = smem + 24;                          // 1 double
  double* ks = smem + 32;                          // D doubles
  const int t = threadIdx.x;

  // Pass 1: total residual T.
  const double T = scan_block_totals(a, u, scr, [](int, double, double) {});
  if (is_init && t == 0) a.T0[u] = T;
  const double T0 = is_init ? T : a.T0[u];
  if (!(T > kStopRel * T0)) { mark_stopped(a, u, i); return; }
  const double target = a.u[(size_t)u * a.r + i] * T;

  // Pass 2: first block whose last prefix exceeds the target.
  int myb = INT_MAX, mypos = -1;
  double myP = 0.0;
  scan_block_totals(a, u, scr, [&](int b, double P, double x) {
    if (P + x > target && b < myb) { myb = b; myP = P; }
    if (x > 0.0) mypos = b;
  });
  const int bstar = block_min_int(myb, iscr);
  const bool fallback = (bstar == INT_MAX);
  const int bsel = fallback ? block_max_int(mypos, iscr) : bstar;
  if (bsel < 0) { mark_stopped(a, u, i); return; }   // no mass at all
  if (!fallback && myb == bstar) *sP = myP;
  __syncthreads();
  const double Pb = fallback ? 0.0 : *sP;

  // Rescan the chosen block exactly as its owner did.
  const double* du = a.dres + (size_t)u * a.npad;
  const int row0 = bsel * RB + t * RPT;
  double v[RPT], ex[RPT], tot;
#pragma unroll
  for (int k = 0; k < RPT; ++k) v[k] = du[row0 + k];
  double dv[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) dv[k] = v[k];
  block_scan<RPT>(v, ex, tot, scr);
  // First index with mass whose prefix exceeds the target; the last index
  // with mass in the block if rounding across lanes leaves none (and always
  // in the fallback case).  Either way s is a valid index with d_s > 0.
  int cand = INT_MAX, lastpos = -1;
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int l = row0 + k;
    if (l < a.n && dv[k] > 0.0) {
      lastpos = l;
      if (!fallback && Pb + v[k] > target && l < cand) cand = l;
    }
  }
  int s = block_min_int(cand, iscr);
  if (s == INT_MAX) s = block_max_int(lastpos, iscr);
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
  const double* Fu = a.F + (size_t)u * a.r * a.npad;
  double* Lrow = a.L + ((size_t)u * a.r + i) * a.r;
  double sq = 0.0;
  for (int j = t; j < a.r; j += kBlock) {
    if (j < i) {
      const double f = Fu[(size_t)j * a.npad + s];
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

// Unit's last workgroup detection: every thread fences its own stores, then
// one atomic per workgroup.  Returns true in all threads of the last one.
__device__ __forceinline__ bool last_block_of_unit(const SelectArgs& a, int u, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&a.counter[u], 1u);
    *flag = (prev == (unsigned)a.nb - 1u) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) {
    __threadfence();
    if (threadIdx.x == 0) a.counter[u] = 0u;
  }
  return last;
}

__global__ __launch_bounds__(kBlock) void rpc_clear(SelectArgs a, int U) {
  const int u = blockIdx.x * kBlock + threadIdx.x;
  if (u < U) {
    a.stopped[u] = 0;
    a.reff[u] = a.r;
    a.counter[u] = 0u;
  }
}

// Per-unit key mean (recentring), fp64, fixed reduction order.
template <typename TK, int D>
__global__ __launch_bounds__(kBlock) void rpc_kbar(SelectArgs a) {
  __shared__ double part[kBlock];
  const int u = blockIdx.x, t = threadIdx.x;
  constexpr int PH = kBlock / D;   // row phases
  const int c = t % D, ph = t / D;
  const TK* K = reinterpret_cast<const TK*>(a.K) + (size_t)u * a.n * D;
  double acc = 0.0;
  for (int l = ph; l < a.n; l += PH) acc += (double)Elem<TK>::f32(K, (size_t)l * D + c);
  part[t] = acc;
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int p = 0; p < PH; ++p) s += part[p * D + t];
    a.kbar[(size_t)u * D + t] = s / (double)a.n;
  }
}

// Residual diagonal h_tau(k_l, k_l), its block totals, and pivot 0.
template <typename TK, int D, bool RC>
__global__ __launch_bounds__(kBlock) void rpc_init(SelectArgs a) {
  extern __shared__ double smem[];
  double* s_kbar = smem + 32 + D;
  __shared__ int flag;
  const int u = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
  if (RC) {
    for (int c = t; c < D; c += kBlock) s_kbar[c] = a.kbar[(size_t)u * D + c];
    __syncthreads();
  }
  const TK* K = reinterpret_cast<const TK*>(a.K) + (size_t)u * a.n * D;
  double* du = a.dres + (size_t)u * a.npad;
  const int row0 = blk * RB + t * RPT;
  double v[RPT], ex[RPT], tot;
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int l = row0 + k;
    v[k] = l < a.n ? exp(a.c * key_sqnorm<TK, D, RC>(K + (size_t)l * D, s_kbar)) : 0.0;
    du[l] = v[k];
  }
  block_scan<RPT>(v, ex, tot, smem);
  if (t == 0) a.bsum[(size_t)u * a.nb + blk] = tot;
  if (!last_block_of_unit(a, u, &flag)) return;
  draw_and_stage<TK, D, RC>(a, u, 0, true, smem);
}

// One RPNys round i for every unit still running.
template <typename TK, int D, bool RC>
__global__ __launch_bounds__(kBlock) void rpc_step(SelectArgs a, int i) {
  extern __shared__ double smem[];
  double* s_ks = smem + 32;            // D
  double* s_kbar = s_ks + D;           // D
  double* s_prow = s_kbar + D;         // r
  __shared__ int flag;
  const int u = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
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

  const int row0 = blk * RB + t * RPT;
  double* Fu = a.F + (size_t)u * a.r * a.npad;
  double* du = a.dres + (size_t)u * a.npad;
  double v[RPT] = {0.0, 0.0}, ex[RPT], tot;
  if (row0 < a.n) {
    // sum_j F[j][l] * F[s][j] for the thread's two rows, 4 partial sums each.
    double p0x = 0.0, p0y = 0.0, p1x = 0.0, p1y = 0.0, p2x = 0.0, p2y = 0.0, p3x = 0.0, p3y = 0.0;
    const double* Fr = Fu + row0;
    const size_t ld = (size_t)a.npad;
    int j = 0;
    for (; j + 4 <= i; j += 4) {
      const double2 f0 = *reinterpret_cast<const double2*>(Fr + (size_t)(j + 0) * ld);
      const double2 f1 = *reinterpret_cast<const double2*>(Fr + (size_t)(j + 1) * ld);
      const double2 f2 = *reinterpret_cast<const double2*>(Fr + (size_t)(j + 2) * ld);
      const double2 f3 = *reinterpret_cast<const double2*>(Fr + (size_t)(j + 3) * ld);
      const double q0 = s_prow[j], q1 = s_prow[j + 1], q2 = s_prow[j + 2], q3 = s_prow[j + 3];
      p0x = fma(f0.x, q0, p0x); p0y = fma(f0.y, q0, p0y);
      p1x = fma(f1.x, q1, p1x); p1y = fma(f1.y, q1, p1y);
      p2x = fma(f2.x, q2, p2x); p2y = fma(f2.y, q2, p2y);
      p3x = fma(f3.x, q3, p3x); p3y = fma(f3.y, q3, p3y);
    }
    for (; j < i; ++j) {
      const double2 f0 = *reinterpret_cast<const double2*>(Fr + (size_t)j * ld);
      const double q0 = s_prow[j];
      p0x = fma(f0.x, q0, p0x); p0y = fma(f0.y, q0, p0y);
    }
    const double accx = (p0x + p1x) + (p2x + p3x);
    const double accy = (p0y + p1y) + (p2y + p3y);

    const TK* K = reinterpret_cast<const TK*>(a.K) + (size_t)u * a.n * D;
    const double gx = exp(a.c * key_dot<TK, D, RC>(K + (size_t)row0 * D, s_ks, s_kbar)) - accx;
    const bool has_y = row0 + 1 < a.n;
    const double gy = has_y ? exp(a.c * key_dot<TK, D, RC>(K + (size_t)(row0 + 1) * D, s_ks, s_kbar)) - accy : 0.0;
    const double fx = gx / sgs;
    const double fy = has_y ? gy / sgs : 0.0;
    *reinterpret_cast<double2*>(Fu + (size_t)i * ld + row0) = make_double2(fx, fy);
    const double2 dold = *reinterpret_cast<const double2*>(du + row0);
    const double fx2 = fx * fx, fy2 = fy * fy;
    double dx = dold.x - fx2, dy = dold.y - fy2;
    dx = dx > 0.0 ? dx : 0.0;
    dy = dy > 0.0 ? dy : 0.0;
    if (row0 == s) { dx = 0.0; a.L[((size_t)u * a.r + i) * a.r + i] = fx; }
    if (row0 + 1 == s) { dy = 0.0; a.L[((size_t)u * a.r + i) * a.r + i] = fy; }
    if (!has_y) dy = 0.0;
    *reinterpret_cast<double2*>(du + row0) = make_double2(dx, dy);
    v[0] = dx;
    v[1] = dy;
  }
  block_scan<RPT>(v, ex, tot, smem);
  if (t == 0) a.bsum[(size_t)u * a.nb + blk] = tot;
  if (!last_block_of_unit(a, u, &flag)) return;
  if (i + 1 < a.r) draw_and_stage<TK, D, RC>(a, u, i + 1, false, smem);
}

// r_eff, -1 padding of S and zero rows of L past r_eff.
__global__ __launch_bounds__(kBlock) void rpc_finalize(SelectArgs a, int32_t* r_eff_out) {
  const int u = blockIdx.x, t = threadIdx.x;
  const int re = a.stopped[u] ? a.reff[u] : a.r;
  if (t == 0) r_eff_out[u] = re;
  for (int j = re + t; j < a.r; j += kBlock) a.S[(size_t)u * a.r + j] = -1;
  double* Lu = a.L + (size_t)u * a.r * a.r;
  const size_t from = (size_t)re * a.r, to = (size_t)a.r * a.r;
  for (size_t e = from + t; e < to; e += kBlock) Lu[e] = 0.0;
}

template <typename TK, int D, bool RC>
static hipError_t launch_select_t(const SelectArgs& a, int U, int32_t* r_eff, hipStream_t st) {
  const dim3 grid(a.nb, U);
  rpc_clear<<<(U + kBlock - 1) / kBlock, kBlock, 0, st>>>(a, U);
  if (RC) rpc_kbar<TK, D><<<U, kBlock, 0, st>>>(a);
  const size_t lds_init = (32 + 2 * D) * sizeof(double);
  rpc_init<TK, D, RC><<<grid, kBlock, lds_init, st>>>(a);
  const size_t lds_step = (32 + 2 * D + a.r) * sizeof(double);
  for (int i = 0; i < a.r; ++i) rpc_step<TK, D, RC><<<grid, kBlock, lds_step, st>>>(a, i);
  rpc_finalize<<<U, kBlock, 0, st>>>(a, r_eff);
  return hipGetLastError();
}

template <typename TK, int D>
static hipError_t launch_select_rc(const SelectArgs& a, int U, bool rc, int32_t* r_eff, hipStream_t st) {
  return rc ? launch_select_t<TK, D, true>(a, U, r_eff, st) : launch_select_t<TK, D, false>(a, U, r_eff, st);
}

template <typename TK>
static hipError_t launch_select_d(const SelectArgs& a, int U, int d, bool rc, int32_t* r_eff, hipStream_t st) {
  switch (d) {
    case 16: return launch_select_rc<TK, 16>(a, U, rc, r_eff, st);
    case 32: return launch_select_rc<TK, 32>(a, U, rc, r_eff, st);
    case 64: return launch_select_rc<TK, 64>(a, U, rc, r_eff, st);
    case 128: return launch_select_rc<TK, 128>(a, U, rc, r_eff, st);
  }
  return hipErrorInvalidValue;
}

// Host entry used by the C ABI (arguments already validated).
hipError_t launch_select(int bf16, int U, int n, int d, int r, double c, int recentre,
                         const void* K, const double* u, int32_t* S, int32_t* r_eff, double* L,
                         void* ws, hipStream_t st) {
  const SelectLayout lay(U, n, d, r);
  char* w = static_cast<char*>(ws);
  SelectArgs a;
  a.K = K; a.u = u; a.S = S; a.L = L;
  a.F = reinterpret_cast<double*>(w + lay.F);
  a.dres = reinterpret_cast<double*>(w + lay.dres);
  a.bsum = reinterpret_cast<double*>(w + lay.bsum);
  a.pivbuf = reinterpret_cast<double*>(w + lay.pivbuf);
  a.T0 = reinterpret_cast<double*>(w + lay.T0);
  a.kbar = reinterpret_cast<double*>(w + lay.kbar);
  a.stopped = reinterpret_cast<int32_t*>(w + lay.stopped);
  a.reff = reinterpret_cast<int32_t*>(w + lay.reff);
  a.counter = reinterpret_cast<uint32_t*>(w + lay.counter);
  a.n = n; a.npad = lay.npad; a.nb = lay.nb; a.r = r; a.pbs = lay.pbs; a.c = c;
  return bf16 ? launch_select_d<bf16_t>(a, U, d, recentre != 0, r_eff, st)
              : launch_select_d<float>(a, U, d, recentre != 0, r_eff, st);
}

}  // namespace wc
