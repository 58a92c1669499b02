// Nystroem weights through the pivot block: X = L^{-T} (L^{-1} Y), float64,
// on the fp64 matrix cores (v_mfma_f64_16x16x4f64).
//
// [WildCat (arXiv 2602.10056), Nystroem and CompressKV / Alg. 2 paragraphs:
// W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K); with h_tau(K_S, K_S) = L L^T from the
// Cholesky pivot block, W [V, 1] = L^{-T} L^{-1} (h_tau(K_S, K) [V, 1]).]
//
// Blocked right-looking solve over diagonal blocks of b rows (b = 64 .. 512,
// chosen from r), each block applied through its explicit inverse:
//   inverses  the 64x64 diagonal blocks of L by substitution (one wave per
//             block), then doubled 64 -> 128 -> .. -> b:
//             inv([[A, 0], [B, C]]) = [[A^-1, 0], [-C^-1 B A^-1, C^-1]],
//             two matrix products per level (T1 = B A^-1, then -C^-1 T1);
//   forward   for t = 0 .. T-1:  Z_t = Dinv_t Y_t;  Y_i -= L_it Z_t (i > t);
//   backward  for t = T-1 .. 0:  X_t = Dinv_t^T Z_t;  Z_i -= L_ti^T X_t (i < t).
// Every step is a product of fp64 tiles: a workgroup owns 16 rows and 16 NC
// columns (NC accumulators of one MFMA each) of one product; its four waves
// split the inner dimension into four ranges, each wave issuing all loads of
// its range (operands straight from global memory in the MFMA lane layout)
// before its MFMAs, and the four partial sums meet in LDS, added in wave
// order.  Summation order per output element is fixed, so the results are
// bitwise reproducible.  The right-hand sides are the d+1 columns of Y padded to a
// multiple of 16 with zeros.
//
// Rows at or beyond r_eff take part as the identity: their rows and columns
// of L read as zero (guarded loads), their diagonal blocks are inverted with
// an identity tail, their rows of Y are zero, so their rows of X come out 0.
//
// Dinv is kept as a band [U][rp][b]: row i holds row i of the inverse of its
// b-block (columns relative to the block start), zero above the diagonal.
//
// XCD-aware launch: workgroups are dispatched to the 8 XCDs round-robin by
// linear index; with at least 8 units, all workgroups of unit u get indices
// with index % 8 == u % 8, so a unit's operands (its block of Z, its panels
// of L) are shared through one XCD's L2.
#include "common.hpp"
#include "ordered.hpp"
#include "weights_layout.hpp"

namespace wc {

typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kXcds = 8;

// One wave: acc[c] += A[0:16][kb:ke] * B[kb:ke][16c : 16c+16], c < NC.
//   A[a][k] = TA ? Ab[k * lda + a] : Ab[a * lda + k]    B[k][j] = Bb[k * ldb + j]
// Lane (r = lane % 16, q = lane / 16) feeds, for MFMA j of each 16-wide k
// chunk, A[r][k0 + 4q + j] and B[k0 + 4q + j][16c + r]: the four MFMAs of a
// chunk together cover k0 .. k0 + 15 (in an order fixed per lane).  Up to PF
// chunks are loaded before their MFMAs (chunk indices past ke re-load the
// last chunk, so every load is unconditional).  With GUARD, A entries with
// a >= alim or k >= klim read as 0 (indices clamped so that every load stays
// in bounds).  kb, ke: multiples of 16.  On return, element v of acc[c] in
// lane (r, q) is row 4v + q, column 16c + r of the product (the output
// layout of this MFMA on gfx950).
template <int NC, bool TA, bool GUARD, int PF>
__device__ __forceinline__ void wave_mma(const double* __restrict__ Ab, int lda, const double* __restrict__ Bb, int ldb,
                                         int kb, int ke, int alim, int klim, f64x4 (&acc)[NC]) {
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
#pragma unroll 1
  for (int k0 = kb; k0 < ke; k0 += 16 * PF) {
    const int nch = min(PF, (ke - k0) / 16);
    double a[PF][4], b[PF][NC][4];
#pragma unroll
    for (int ch = 0; ch < PF; ++ch) {
      const int kc = k0 + 16 * min(ch, nch - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = kc + 4 * q + j;
        if (GUARD) {
          const int kk = max(min(k, klim - 1), 0), rr = max(min(r, alim - 1), 0);
          const double v = TA ? Ab[(size_t)kk * lda + rr] : Ab[(size_t)rr * lda + kk];
          a[ch][j] = (k < klim && r < alim) ? v : 0.0;
        } else {
          a[ch][j] = TA ? Ab[(size_t)k * lda + r] : Ab[(size_t)r * lda + k];
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) b[ch][c][j] = Bb[(size_t)k * ldb + 16 * c + r];
      }
    }
#pragma unroll
    for (int ch = 0; ch < PF; ++ch) {
      if (ch < nch) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int c = 0; c < NC; ++c)
            acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ch][j], b[ch][c][j], acc[c], 0, 0, 0);
      }
    }
  }
}

template <int NC> constexpr int prefetch_chunks() { return NC >= 5 ? 2 : 4; }

// Partial sums of waves 1..3 of a workgroup, [wave - 1][c][v][lane].
template <int NC> struct RedLds { double v[3 * NC * 4 * 64]; };

// Workgroup: acc (valid in wave 0 on return) = A[0:16][kb:ke] B[kb:ke][..],
// the chunks of [kb, ke) split into four contiguous ranges, one per wave,
// and the partials added in wave order.  Every wave of the workgroup must
// call it (it synchronises the workgroup).
template <int NC, bool TA, bool GUARD>
__device__ __forceinline__ void wg_mma(const double* __restrict__ Ab, int lda, const double* __restrict__ Bb, int ldb,
                                       int kb, int ke, int alim, int klim, f64x4 (&acc)[NC], RedLds<NC>& red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = ke > kb ? (ke - kb) / 16 : 0;
  const int per = (nch + 3) / 4;
  const int c0 = min(nch, wave * per), c1 = min(nch, c0 + per);
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
  wave_mma<NC, TA, GUARD, prefetch_chunks<NC>()>(Ab, lda, Bb, ldb, kb + 16 * c0, kb + 16 * c1, alim, klim, acc);
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) red.v[(((wave - 1) * NC + c) * 4 + v) * 64 + lane] = acc[c][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][v] += red.v[((w * NC + c) * 4 + v) * 64 + lane];
  }
}

// Workgroup placement: (unit, tile) of linear workgroup index `id`, with
// `per` tiles per unit.  Returns false for padding workgroups.
__device__ __forceinline__ bool place(int id, int per, int U, int& unit, int& tile) {
  if (U >= kXcds) {
    const int xcd = id % kXcds, slot = id / kXcds;
    unit = (slot / per) * kXcds + xcd;
    tile = slot % per;
  } else {
    unit = id / per;
    tile = id % per;
  }
  return unit < U;
}

static inline unsigned grid_for(int per, int U) {
  return (unsigned)(U >= kXcds ? (U + kXcds - 1) / kXcds * kXcds * per : U * per);
}

struct SolveArgs {
  const float* ypart;   // [nsplit][U][r][D1] split-n partials of Y
  const double* L;      // [U][r][r]
  const int32_t* r_eff;
  double* band;         // [U][rp][b] inverses of the diagonal blocks
  double* T1;           // [U][rp/2][b/2] doubling scratch
  double* Y;            // [U][rp][cp] right-hand sides, then X (fp64)
  double* Z;            // [U][rp][cp]
  float* X;             // [U][r][D1] output
  const int* mmslot;    // [U][2][d] order-encoded column min / max of V
  float *vmin, *vmax;   // [U][d] output
  int nsplit, U, r, rp, b, D1, cp;
};

// Y[u][i][c] = sum of the split partials in split order (fp64), 0 for rows
// at or past r_eff and for the padding columns.  The first U d threads also
// decode the value range of V (one launch fewer).
__global__ __launch_bounds__(kBlock) void solve_prep(SolveArgs a) {
  const size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x;
  const int d = a.D1 - 1;
  if (e < (size_t)a.U * d) {
    const int u = (int)(e / d), c = (int)(e % d);
    a.vmin[e] = ord_dec(a.mmslot[((size_t)u * 2) * d + c]);
    a.vmax[e] = ord_dec(a.mmslot[((size_t)u * 2 + 1) * d + c]);
  }
  const size_t per = (size_t)a.rp * a.cp;
  if (e >= per * a.U) return;
  const int u = (int)(e / per);
  const int i = (int)((e % per) / a.cp), c = (int)(e % a.cp);
  const bool live = i < a.r_eff[u] && c < a.D1;
  const size_t split = (size_t)a.U * a.r * a.D1;
  const float* p = a.ypart + ((size_t)u * a.r + min(i, a.r - 1)) * a.D1 + min(c, a.D1 - 1);
  double z = 0.0;
  for (int s0 = 0; s0 < a.nsplit; s0 += 8) {   // 8 loads in flight, added in split order
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[(size_t)min(s0 + k, a.nsplit - 1) * split];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < a.nsplit) z += (double)v[k];
  }
  a.Y[e] = live ? z : 0.0;
}

// Inverse of the 64x64 diagonal block `blk` of L[u] (identity past r_eff),
// into the band; the band columns to its right in the same rows are zeroed.
// One wave per block, lane j computes column j of the inverse by column-
// oriented substitution from e_j: step m removes row m's value from the rows
// below, b_i -= (L_im / L_mm) b_m (i > m), and at the end x_m = b_m / L_mm.
// The block sits transposed and pre-scaled in LDS (Sc[m][i] = L_im / L_mm,
// Sc[m][m] = 1 / L_mm), so step m reads the contiguous row m of Sc; those
// reads do not depend on b and are issued one step ahead, in a batch
// (scheduling barriers keep the batch together), and the only dependency
// from step to step is one FMA.
__global__ __launch_bounds__(64) void solve_inv64(SolveArgs a) {
  __shared__ __attribute__((aligned(16))) double Sc[64 * 64];
  const int blk = blockIdx.x, u = blockIdx.y, j = threadIdx.x;
  const int i0 = blk * 64, re = a.r_eff[u];
  const int nt = max(0, min(64, re - i0));
  const double* Lu = a.L + (size_t)u * a.r * a.r;
  // lane j stages column j of the block, scaled: Sc[j][i] = L[i][j] / L[j][j]
  // for i > j and Sc[j][j] = 1 / L[j][j] (identity past r_eff); all loads
  // (row i: consecutive lanes, consecutive addresses) are issued before the
  // first LDS store, and the scaling happens in registers
  {
    double v[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = Lu[(size_t)min(i0 + i, a.r - 1) * a.r + min(i0 + j, a.r - 1)];
    const double dj = Lu[(size_t)min(i0 + j, a.r - 1) * a.r + min(i0 + j, a.r - 1)];
    const double rinv = 1.0 / (j < nt ? dj : 1.0);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const double x = (i < nt && j < nt) ? v[i] : 0.0;   // below the diagonal only i > j is read
      Sc[j * 64 + i] = i == j ? rinv : x * rinv;
    }
  }
  __syncthreads();
  double b[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) b[i] = i == j ? 1.0 : 0.0;
  double cur[64], nxt[64];
#pragma unroll
  for (int i = 1; i < 64; ++i) cur[i] = Sc[i];
#pragma unroll
  for (int m = 0; m < 63; ++m) {
#pragma unroll
    for (int i = m + 2; i < 64; ++i) nxt[i] = Sc[(m + 1) * 64 + i];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = m + 1; i < 64; ++i) b[i] = fma(-cur[i], b[m], b[i]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = m + 2; i < 64; ++i) cur[i] = nxt[i];
  }
  const int col0 = i0 % a.b;   // the block's columns within its b-block
  double* Bu = a.band + ((size_t)u * a.rp + i0) * a.b;
#pragma unroll
  for (int i = 0; i < 64; ++i) Bu[(size_t)i * a.b + col0 + j] = b[i] * Sc[i * 64 + i];
  for (int i = 0; i < 64; ++i)
    for (int c = col0 + 64 + j; c < a.b; c += 64) Bu[(size_t)i * a.b + c] = 0.0;
}

// Doubling, level s -> 2s, pair p of unit u (rows [2ps, 2ps + 2s)):
//   T1 = B A^-1,  B = L[(2p+1)s + a][2ps + k],  A^-1 = band block at rows 2ps.
// Workgroup tile: 16 rows x 16 NC columns of the s x s product.
template <int NC>
__global__ __launch_bounds__(256) void solve_dbl_t1(SolveArgs a, int s) {
  __shared__ RedLds<NC> red;
  const int rt = s / 16, cg = s / (16 * NC), per = rt * cg * (a.rp / (2 * s));
  int u, tile;
  if (!place(blockIdx.x, per, a.U, u, tile)) return;
  const int p = tile / (rt * cg), rem = tile % (rt * cg), ti = rem / cg, gj = rem % cg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int re = a.r_eff[u];
  const int rowA = (2 * p + 1) * s + 16 * ti;   // first row of L (and of the product, + offset)
  const int colL = 2 * p * s;                   // column of L where B starts
  const int c0 = 16 * NC * gj;
  const bool live = rowA < re && colL < re;
  const double* Lb = a.L + (size_t)u * a.r * a.r + (size_t)min(rowA, a.r - 1) * a.r + min(colL, a.r - 1);
  const double* Ainv = a.band + ((size_t)u * a.rp + colL) * a.b + (colL % a.b) + c0;
  f64x4 acc[NC];
  // A^-1 is lower triangular: rows k < c0 of its column group are zero
  wg_mma<NC, false, true>(Lb, a.r, Ainv, a.b, c0 & ~15, live ? s : 0, re - rowA, re - colL, acc, red);
  if (wave != 0) return;
  double* T = a.T1 + ((size_t)u * (a.rp / 2) + (size_t)p * s + 16 * ti) * (a.b / 2) + c0;
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) T[(size_t)(4 * v + q) * (a.b / 2) + 16 * c + r16] = acc[c][v];
}

//   band[(2p+1)s + a][2ps - tb + c] = -(C^-1 T1)[a][c],  C^-1 = band block at rows (2p+1)s.
template <int NC>
__global__ __launch_bounds__(256) void solve_dbl_x21(SolveArgs a, int s) {
  __shared__ RedLds<NC> red;
  const int rt = s / 16, cg = s / (16 * NC), per = rt * cg * (a.rp / (2 * s));
  int u, tile;
  if (!place(blockIdx.x, per, a.U, u, tile)) return;
  const int p = tile / (rt * cg), rem = tile % (rt * cg), ti = rem / cg, gj = rem % cg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ar = 16 * ti;                       // row within C
  const int row = (2 * p + 1) * s + ar;         // row of the band
  const int c0 = 16 * NC * gj;
  const double* Cinv = a.band + ((size_t)u * a.rp + row) * a.b + (((2 * p + 1) * s) % a.b);
  const double* T = a.T1 + ((size_t)u * (a.rp / 2) + (size_t)p * s) * (a.b / 2) + c0;
  f64x4 acc[NC];
  // C^-1 lower triangular: rows [ar, ar + 16) need k < ar + 16
  wg_mma<NC, false, false>(Cinv, a.b, T, a.b / 2, 0, ar + 16, 0, 0, acc, red);
  if (wave != 0) return;
  double* out = a.band + ((size_t)u * a.rp + row) * a.b + ((2 * p * s) % a.b) + c0;
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(size_t)(4 * v + q) * a.b + 16 * c + r16] = -acc[c][v];
}

// Diagonal block t of a sweep.  Forward (BWD = false): Z_t = Dinv_t Y_t.
// Backward: X_t = Dinv_t^T Z_t, written to the fp64 X (aliasing Y) and to the
// float32 output (rows < r; 0 at or past r_eff).  Workgroup tile: 16 rows x
// 16 NC columns; a block past r_eff only writes its zero rows.
template <int NC, bool BWD>
__global__ __launch_bounds__(256) void solve_diag(SolveArgs a, int t) {
  __shared__ RedLds<NC> red;
  const int G = a.cp / (16 * NC), rt = a.b / 16, per = rt * G;
  int u, tile;
  if (!place(blockIdx.x, per, a.U, u, tile)) return;
  const int ti = tile / G, gj = tile % G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int tb = t * a.b, re = a.r_eff[u];
  const int ar = 16 * ti;   // row within the block
  const int c0 = 16 * NC * gj;
  const bool live = tb < re;
  const double* Bd = a.band + ((size_t)u * a.rp + tb + ar) * a.b;
  f64x4 acc[NC];
  if (!BWD) {
    const double* In = a.Y + ((size_t)u * a.rp + tb) * a.cp + c0;
    wg_mma<NC, false, false>(Bd, a.b, In, a.cp, 0, live ? ar + 16 : 0, 0, 0, acc, red);
  } else {
    const double* In = a.Z + ((size_t)u * a.rp + tb + ar) * a.cp + c0;
    // (Dinv^T)[a][k] = Dinv[k][a], nonzero for k >= a
    wg_mma<NC, true, false>(Bd + ar, a.b, In, a.cp, 0, live ? a.b - ar : 0, 0, 0, acc, red);
  }
  if (wave != 0) return;
  double* Out = (BWD ? a.Y : a.Z) + ((size_t)u * a.rp + tb + ar) * a.cp + c0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) Out[(size_t)(4 * v + q) * a.cp + 16 * c + r16] = acc[c][v];
  if (BWD) {
    float* Xu = a.X + (size_t)u * a.r * a.D1;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = tb + ar + 4 * v + q;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = c0 + 16 * c + r16;
        if (i < a.r && col < a.D1) Xu[(size_t)i * a.D1 + col] = i < re ? (float)acc[c][v] : 0.0f;
      }
    }
  }
}

// Trailing update after block t.  Forward: Y_i -= L[i][tb + k] Z_t[k] for
// rows i >= tb + b; backward: Z_i -= L[tb + k][i] X_t[k] for rows i < tb.
// Only rows and k below r_eff take part.  Workgroup tile: 16 rows x 16 NC
// columns.
template <int NC, bool BWD>
__global__ __launch_bounds__(256) void solve_update(SolveArgs a, int t) {
  __shared__ RedLds<NC> red;
  const int tb = t * a.b;
  const int row0 = BWD ? 0 : tb + a.b;
  const int nrows = BWD ? tb : a.rp - row0;
  const int G = a.cp / (16 * NC), rt = nrows / 16, per = rt * G;
  int u, tile;
  if (!place(blockIdx.x, per, a.U, u, tile)) return;
  const int ti = tile / G, gj = tile % G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int re = a.r_eff[u];
  const int i0 = row0 + 16 * ti;
  if (i0 >= re || tb >= re) return;   // whole workgroup: rows past r_eff stay 0, a block past r_eff adds nothing
  const int c0 = 16 * NC * gj;
  const int kl = min(a.b, re - tb);     // k < kl take part
  const int ke = (kl + 15) & ~15;
  const double* Lu = a.L + (size_t)u * a.r * a.r;
  const double* Bk = (BWD ? a.Y : a.Z) + ((size_t)u * a.rp + tb) * a.cp + c0;
  const bool full = kl == a.b && i0 + 16 <= re;
  f64x4 acc[NC];
  if (!BWD) {
    const double* Ab = Lu + (size_t)min(i0, a.r - 1) * a.r + tb;
    if (full) wg_mma<NC, false, false>(Ab, a.r, Bk, a.cp, 0, ke, 0, 0, acc, red);
    else wg_mma<NC, false, true>(Ab, a.r, Bk, a.cp, 0, ke, re - i0, kl, acc, red);
  } else {
    const double* Ab = Lu + (size_t)tb * a.r + i0;
    if (full) wg_mma<NC, true, false>(Ab, a.r, Bk, a.cp, 0, ke, 0, 0, acc, red);
    else wg_mma<NC, true, true>(Ab, a.r, Bk, a.cp, 0, ke, re - i0, kl, acc, red);
  }
  if (wave != 0) return;
  double* C = (BWD ? a.Z : a.Y) + ((size_t)u * a.rp + i0) * a.cp + c0;
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double* y = C + (size_t)(4 * v + q) * a.cp + 16 * c + r16;
      *y -= acc[c][v];
    }
}

template <int NC>
static void launch_sweeps(const SolveArgs& a, const SolveGeom& g, hipStream_t st) {
  const int G = g.cp / (16 * NC);
  const int T = g.rp / g.b;
  for (int t = 0; t < T; ++t) {
    solve_diag<NC, false><<<grid_for((g.b / 16) * G, a.U), 256, 0, st>>>(a, t);
    const int nrows = g.rp - (t + 1) * g.b;
    if (nrows > 0) solve_update<NC, false><<<grid_for((nrows / 16) * G, a.U), 256, 0, st>>>(a, t);
  }
  for (int t = T - 1; t >= 0; --t) {
    solve_diag<NC, true><<<grid_for((g.b / 16) * G, a.U), 256, 0, st>>>(a, t);
    const int nrows = t * g.b;
    if (nrows > 0) solve_update<NC, true><<<grid_for((nrows / 16) * G, a.U), 256, 0, st>>>(a, t);
  }
}

// X = L^{-T} L^{-1} (sum of the split partials of Y), for every unit; also
// decodes the value range (vmin, vmax) gathered by value_range_part.
hipError_t launch_trsm(int U, int r, int d, const float* ypart, int nsplit, const double* L, const int32_t* r_eff,
                       float* X, float* vmin, float* vmax, const WeightsLayout& lay, char* ws, hipStream_t st) {
  const SolveGeom& g = lay.sg;
  SolveArgs a{};
  a.ypart = ypart; a.L = L; a.r_eff = r_eff; a.X = X;
  a.mmslot = reinterpret_cast<const int*>(ws + lay.mmslot); a.vmin = vmin; a.vmax = vmax;
  a.band = reinterpret_cast<double*>(ws + lay.band);
  a.T1 = reinterpret_cast<double*>(ws + lay.t1);
  a.Y = reinterpret_cast<double*>(ws + lay.yw);
  a.Z = reinterpret_cast<double*>(ws + lay.zw);
  a.nsplit = nsplit; a.U = U; a.r = r; a.rp = g.rp; a.b = g.b; a.D1 = d + 1; a.cp = g.cp;
  const size_t ny = (size_t)U * g.rp * g.cp;
  solve_prep<<<(unsigned)((ny + kBlock - 1) / kBlock), kBlock, 0, st>>>(a);
  solve_inv64<<<dim3(g.rp / 64, U), 64, 0, st>>>(a);
  for (int s = 64; s < g.b; s *= 2) {
    const int pairs = g.rp / (2 * s), per = (s / 16) * (s / 64) * pairs;
    solve_dbl_t1<4><<<grid_for(per, U), 256, 0, st>>>(a, s);
    solve_dbl_x21<4><<<grid_for(per, U), 256, 0, st>>>(a, s);
  }
  switch (g.nc) {
    case 2: launch_sweeps<2>(a, g, st); break;
    case 3: launch_sweeps<3>(a, g, st); break;
    case 5: launch_sweeps<5>(a, g, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace wc
