// Nystroem weights through the pivot block: X = L^{-T} (L^{-1} Y), float64,
// on the fp64 matrix cores (v_mfma_f64_16x16x4f64).
//
// [WildCat (arXiv 2602.10056), Nystroem and CompressKV / Alg. 2 paragraphs:
// W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K); with h_tau(K_S, K_S) = L L^T from the
// Cholesky pivot block, W [V, 1] = L^{-T} L^{-1} (h_tau(K_S, K) [V, 1]).]
//
// Blocked right-looking solve over diagonal blocks of b rows (b = 64 .. 256,
// chosen from r), each block applied through its explicit inverse:
//   inverses  the 64x64 diagonal blocks of L, each in one workgroup's LDS by
//             doubling from 16x16 blocks (launched together with the sum of
//             the split partials of Y), then doubled 64 -> 128 -> .. -> b,
//             one launch per level:
//             inv([[A, 0], [B, C]]) = [[A^-1, 0], [-C^-1 B A^-1, C^-1]]
//             (T1 = B A^-1, then -C^-1 T1, column slab by column slab);
//   forward   for t = 0 .. T-1:  Z_t = Dinv_t Y_t;  Y_i -= L_it Z_t (i > t);
//   backward  for t = T-1 .. 0:  X_t = Dinv_t^T Z_t;  Z_i -= L_ti^T X_t (i < t).
// Every sweep step is a product of fp64 tiles: a workgroup owns 16 rows and 16 NC
// columns (NC accumulators of one MFMA each) of one product; its four waves
// split the inner dimension into four ranges, each wave loading its range in
// batches of a few 16-wide chunks (operands straight from global memory in
// the MFMA lane layout), each batch issued before its MFMAs, and the four
// partial sums meet in LDS, added in wave order.  Summation order per output element is fixed, so the results are
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

// Chunks per batch of loads.  Two for NC >= 3: fewer values in flight per
// wave, but a third wave per SIMD (measured faster than four).
template <int NC> constexpr int prefetch_chunks() { return NC >= 3 ? 2 : 4; }

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
  double* Y;            // [U][rp][cp] right-hand sides, then X (fp64)
  double* Z;            // [U][rp][cp]
  float* X;             // [U][r][D1] output
  const int* mmslot;    // [U][2][d] order-encoded column min / max of V
  float *vmin, *vmax;   // [U][d] output
  int nsplit, U, r, rp, b, D1, cp;
};

// Front of the solve, one launch with two roles:
//  * the first U (rp / 64) workgroups invert the 64x64 diagonal blocks of L
//    (identity past r_eff) into the band, and zero the band columns to the
//    right of each block within its b-block;
//  * the others form Y[u][i][c] = the sum of the split partials in split
//    order (fp64; 0 for rows at or past r_eff and for the padding columns)
//    and decode the value range of V.
// Inversion of a 64x64 block, in LDS, by doubling from 16x16 blocks:
//   16x16 diagonal blocks  substitution, lane j of wave w computing column j
//                          of block w: x_i = (delta_ij - sum_{m<i} L_im x_m) / L_ii;
//   16 -> 32 -> 64         inv([[A, 0], [B, C]]) = [[A^-1, 0], [-C^-1 B A^-1, C^-1]],
//                          T1 = B A^-1 and X21 = -C^-1 T1 on v_mfma_f64_16x16x4f64.
// The MFMA output of T1 (lane (r, q), element v = row 4v + q, column r) is
// already the B operand of the k-step v of the next product, so within a
// 16x16 tile T1 never leaves the registers.
constexpr int kInvPitch = 65;   // doubles per LDS row of the staged block

constexpr int kFrontLds = 2 * 64 * kInvPitch + 32 * 33;   // doubles of LDS the front launch uses

__device__ __forceinline__ void invert64(const SolveArgs& a, int u, int blk, double* lds) {
  double* const Ls = lds;
  double* const Inv = lds + 64 * kInvPitch;
  double* const T1s = lds + 2 * 64 * kInvPitch;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, r16 = lane & 15, q = lane >> 4;
  const int i0 = blk * 64, re = a.r_eff[u];
  const int nt = max(0, min(64, re - i0));
  const double* Lu = a.L + (size_t)u * a.r * a.r;
  {
    double v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = t + kBlock * k, i = e >> 6, j = e & 63;
      v[k] = (i < nt && j <= i) ? Lu[(size_t)(i0 + i) * a.r + i0 + j] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = t + kBlock * k, i = e >> 6, j = e & 63;
      Ls[i * kInvPitch + j] = (i >= nt && i == j) ? 1.0 : v[k];
    }
  }
  __syncthreads();
  // 16x16 diagonal blocks
  if (lane < 16) {
    const int o = 16 * wave, j = lane;
    double x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double s = i == j ? 1.0 : 0.0;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fma(-Ls[(o + i) * kInvPitch + o + m], x[m], s);
      x[i] = s / Ls[(o + i) * kInvPitch + o + i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Inv[(o + i) * kInvPitch + o + j] = x[i];
  }
  __syncthreads();
  // 16 -> 32: wave p takes the pair of blocks at rows 32p
  if (wave < 2) {
    const int o = 32 * wave;
    f64x4 tt = {0.0, 0.0, 0.0, 0.0}, x = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      tt = __builtin_amdgcn_mfma_f64_16x16x4f64(Ls[(o + 16 + r16) * kInvPitch + o + 4 * kk + q],
                                                Inv[(o + 4 * kk + q) * kInvPitch + o + r16], tt, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      x = __builtin_amdgcn_mfma_f64_16x16x4f64(Inv[(o + 16 + r16) * kInvPitch + o + 16 + 4 * kk + q], tt[kk], x, 0,
                                               0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) Inv[(o + 16 + 4 * v + q) * kInvPitch + o + r16] = -x[v];
  }
  __syncthreads();
  // 32 -> 64: wave w owns the 16x16 tile (w / 2, w % 2) of T1 and of X21
  {
    const int it = wave >> 1, jt = wave & 1;
    f64x4 tt = {0.0, 0.0, 0.0, 0.0};
    // A^-1 lower triangular: column tile jt needs k >= 16 jt
#pragma unroll
    for (int kk = 4 * jt; kk < 8; ++kk)
      tt = __builtin_amdgcn_mfma_f64_16x16x4f64(Ls[(32 + 16 * it + r16) * kInvPitch + 4 * kk + q],
                                                Inv[(4 * kk + q) * kInvPitch + 16 * jt + r16], tt, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) T1s[(16 * it + 4 * v + q) * 33 + 16 * jt + r16] = tt[v];
    __syncthreads();
    f64x4 x = {0.0, 0.0, 0.0, 0.0};
    // C^-1 lower triangular: row tile it needs k < 16 (it + 1)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      if (kk < 4 * (it + 1))
        x = __builtin_amdgcn_mfma_f64_16x16x4f64(Inv[(32 + 16 * it + r16) * kInvPitch + 32 + 4 * kk + q],
                                                 T1s[(4 * kk + q) * 33 + 16 * jt + r16], x, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) Inv[(32 + 16 * it + 4 * v + q) * kInvPitch + 16 * jt + r16] = -x[v];
  }
  __syncthreads();
  // into the band (zero above the diagonal), then the band columns to the right
  const int col0 = i0 % a.b;
  double* Bu = a.band + ((size_t)u * a.rp + i0) * a.b;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = t + kBlock * k, i = e >> 6, j = e & 63;
    Bu[(size_t)i * a.b + col0 + j] = j <= i ? Inv[i * kInvPitch + j] : 0.0;
  }
  const int wr = a.b - col0 - 64;   // band columns to the right of the block in its b-block
  for (int e = t; e < 64 * wr; e += kBlock) Bu[(size_t)(e / wr) * a.b + col0 + 64 + e % wr] = 0.0;
}

__global__ __launch_bounds__(kBlock) void solve_front(SolveArgs a, int ninv, int nprep) {
  __shared__ __attribute__((aligned(16))) double lds[kFrontLds];
  if ((int)blockIdx.x < ninv) {
    const int nb = a.rp / 64;
    invert64(a, blockIdx.x / nb, blockIdx.x % nb, lds);
    return;
  }
  const int d = a.D1 - 1;
  const size_t per = (size_t)a.rp * a.cp, ny = per * a.U, step = (size_t)nprep * kBlock;
  const size_t split = (size_t)a.U * a.r * a.D1;
  for (size_t e = (size_t)(blockIdx.x - ninv) * kBlock + threadIdx.x; e < ny; e += step) {
    if (e < (size_t)a.U * d) {
      const int u = (int)(e / d), c = (int)(e % d);
      a.vmin[e] = ord_dec(a.mmslot[((size_t)u * 2) * d + c]);
      a.vmax[e] = ord_dec(a.mmslot[((size_t)u * 2 + 1) * d + c]);
    }
    const int u = (int)(e / per);
    const int i = (int)((e % per) / a.cp), c = (int)(e % a.cp);
    const bool live = i < a.r_eff[u] && c < a.D1;
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
}

// Doubling, level S -> 2S, pair p of unit u (rows [2pS, 2pS + 2S) of a
// b-block): the lower-left block of the pair's inverse, -C^-1 B A^-1, with
//   B = L[(2p+1)S + i][2pS + k],  A^-1, C^-1 = the band blocks at rows 2pS, (2p+1)S.
// Its columns are independent, so a workgroup owns one slab of 16 columns
// and the whole level is one launch.  Wave w owns row tile w of both
// products:
//   T1 = B A^-1[:, slab]       (S x 16; A^-1 lower triangular, so k starts
//                               at the slab), into LDS;
//   X21[:, slab] = -C^-1 T1    (C^-1 lower triangular: row tile w needs
//                               k < 16 (w + 1)).
// Every global load (the wave's rows of B and of C^-1, and its share of the
// slab of A^-1, which goes to LDS) is issued at the start, so the launch
// waits on memory once.
template <int S>
__global__ __launch_bounds__(4 * S) void solve_dbl(SolveArgs a) {
  static_assert(S == 64 || S == 128, "levels of 64 and 128 rows");
  constexpr int NT = 4 * S;              // threads: one wave per row tile
  constexpr int NCH = S / 16;            // chunks of 16 k
  constexpr int NST = (16 * S + NT - 1) / NT;
  __shared__ double Bs[S * 16];
  __shared__ double T1s[S * 16];
  const int per = (a.rp / (2 * S)) * NCH;
  int u, tile;
  if (!place(blockIdx.x, per, a.U, u, tile)) return;
  const int p = tile / NCH, c = tile % NCH;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  const int re = a.r_eff[u];
  const int colL = 2 * p * S, rowB = (2 * p + 1) * S;
  const int rowA = rowB + 16 * wave;
  // B rows (zero past r_eff; indices clamped into the unit's L)
  const double* Lu = a.L + (size_t)u * a.r * a.r;
  const int ra = min(rowA + r16, re - 1);
  double bl[NCH][4];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 16 * ch + 4 * q + j;
      const bool in = ch >= c && rowA + r16 < re && colL + k < re;
      const double v = Lu[(size_t)max(ra, 0) * a.r + max(min(colL + k, re - 1), 0)];
      bl[ch][j] = in ? v : 0.0;
    }
  // C^-1 rows of the wave's row tile
  const double* Cinv = a.band + ((size_t)u * a.rp + rowB + 16 * wave + r16) * a.b + (rowB % a.b);
  double cx[NCH][4];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int j = 0; j < 4; ++j) cx[ch][j] = ch <= wave ? Cinv[16 * ch + 4 * q + j] : 0.0;
  // the slab of A^-1, rows k >= 16 c
  const double* Ainv = a.band + ((size_t)u * a.rp + colL) * a.b + (colL % a.b) + 16 * c;
  double st[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int e = 256 * c + threadIdx.x + NT * i;
    st[i] = e < 16 * S ? Ainv[(size_t)(e >> 4) * a.b + (e & 15)] : 0.0;
  }
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int e = 256 * c + threadIdx.x + NT * i;
    if (e < 16 * S) Bs[e] = st[i];
  }
  __syncthreads();
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
    if (ch >= c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(bl[ch][j], Bs[(16 * ch + 4 * q + j) * 16 + r16], acc, 0, 0, 0);
#pragma unroll
  for (int v = 0; v < 4; ++v) T1s[(16 * wave + 4 * v + q) * 16 + r16] = acc[v];
  __syncthreads();
  acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
    if (ch <= wave)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(cx[ch][j], T1s[(16 * ch + 4 * q + j) * 16 + r16], acc, 0, 0, 0);
  double* out = a.band + ((size_t)u * a.rp + rowB + 16 * wave) * a.b + (colL % a.b) + 16 * c;
#pragma unroll
  for (int v = 0; v < 4; ++v) out[(size_t)(4 * v + q) * a.b + r16] = -acc[v];
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
  // wave 0 reads the tile it updates before the product, so that read's
  // latency overlaps the operand loads
  double* C = (BWD ? a.Z : a.Y) + ((size_t)u * a.rp + i0) * a.cp + 16 * NC * gj;
  const int r16 = lane & 15, q = lane >> 4;
  double cur[NC][4];
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) cur[c][v] = C[(size_t)(4 * v + q) * a.cp + 16 * c + r16];
  }
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
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) C[(size_t)(4 * v + q) * a.cp + 16 * c + r16] = cur[c][v] - acc[c][v];
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
  a.Y = reinterpret_cast<double*>(ws + lay.yw);
  a.Z = reinterpret_cast<double*>(ws + lay.zw);
  a.nsplit = nsplit; a.U = U; a.r = r; a.rp = g.rp; a.b = g.b; a.D1 = d + 1; a.cp = g.cp;
  // front: the block inverses, and summing workgroups to make about two per
  // CU with them (the summing role loops over Y)
  const int ninv = U * (g.rp / 64);
  const int nprep = ninv < 384 ? 512 - ninv : 128;
  solve_front<<<(unsigned)(ninv + nprep), kBlock, 0, st>>>(a, ninv, nprep);
  for (int s = 64; s < g.b; s *= 2) {
    const unsigned grid = grid_for((g.rp / (2 * s)) * (s / 16), U);
    if (s == 64) solve_dbl<64><<<grid, 4 * 64, 0, st>>>(a);
    else solve_dbl<128><<<grid, 4 * 128, 0, st>>>(a);
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
