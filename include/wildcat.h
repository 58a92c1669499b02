/*
 * wildcat.h -- C ABI of the WildCat weighted-coreset attention library
 * (libwildcat.so, HIP for gfx950 / MI355X).
 *
 * Method: "WildCat: Near-Linear Attention in Theory and Practice"
 * (Schroeder & Mackey, arXiv 2602.10056).  Softmax attention
 * O = diag(A 1)^{-1} A V with A = exp(beta Q K^T) is approximated by attending
 * over a weighted coreset of r keys:
 *   wildcat_select  -- RPNys (Alg. 1): randomly pivoted partial Cholesky of
 *                      H = h_tau(K, K) picks the pivots S and the pivot block L;
 *   wildcat_weights -- CompressKV (Alg. 2): X = W [V, 1] with
 *                      W = h_tau(K_S, K_S)^{-1} h_tau(K_S, K), solved through L,
 *                      plus the column value range of V;
 *   wildcat_attend  -- WtdAttn (Alg. 3): O_hat = diag(U w)^{-1} U V_S with
 *                      U = h(Q, K_S), each entry clipped to [v_min j, v_max j].
 * Calling the three in order on one stream is the WildCat module (Alg. 4).
 *   wildcat_decode  -- generation over the cache: m new tokens attend to the
 *                      coreset and, causally, to each other.
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless a comment says "host".
 *  - Tensors are dense, row-major, with the head dimension fastest:
 *      K, V  [batch][kv_heads][n][d]      Q, O  [batch][q_heads][m][d]
 *    A "unit" is one (batch, kv_head) pair, U = batch * kv_heads; unit
 *    u = b * kv_heads + h.  Query head h of batch b reads unit
 *    b * kv_heads + h / (q_heads / kv_heads) (contiguous GQA groups).
 *  - The caller allocates and owns every buffer, including the workspace
 *    whose size the *_workspace_bytes queries return.  The library allocates
 *    no device memory.  Its only state is, per device, a pool of sets of
 *    auxiliary default-priority streams and events, and the static scratch
 *    of wildcat_decode_noalloc.  wildcat_select splits the units into
 *    groups, forks the groups onto one set's streams with an event recorded
 *    on `stream`, and joins them back into `stream` before it returns, so the
 *    call stays ordered on `stream` like any other; a call holds its set only
 *    while it enqueues, concurrent calls take different sets (a set is
 *    created when all are taken; sets are kept until the process ends).
 *    Calls are re-entrant as long as concurrent calls use distinct outputs and
 *    workspaces (wildcat_decode_noalloc: see there).
 *  - Every call only enqueues kernels on `stream` and returns; results are
 *    ready when the stream is synchronised.  A status is returned at once for
 *    argument, shape, dtype and workspace problems; those are checked on the
 *    host before anything is launched.  WILDCAT_ERR_HIP reports a failed
 *    launch; faults during execution surface at the caller's next sync.
 *  - Data conditions are not errors: when the residual trace falls to
 *    1e-12 of its initial value (or is not finite), or the residual at a
 *    drawn pivot is not positive, selection stops early with r_eff < r.
 *    Entries of S past r_eff are -1, rows of L, K_S and X past r_eff are 0
 *    (such rows contribute nothing to wildcat_attend).
 *  - Input values must be finite, and beta*<x,y>/tau^2 must stay inside the
 *    float32 exp range (|.| < 88) for key/key and query/key pairs; the
 *    library does not rescale.  Larger values give inf/NaN intermediates and
 *    clipped garbage outputs, not an error status, from the asynchronous
 *    calls; wildcat_check_range checks this contract on the data (host-
 *    synchronous) and returns WILDCAT_ERR_RANGE when it does not hold.
 */
#ifndef WILDCAT_H
#define WILDCAT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WILDCAT_OK = 0,
  WILDCAT_ERR_ARG = -1,        /* null pointer, non-finite or non-positive beta/tau */
  WILDCAT_ERR_DTYPE = -2,      /* dtype not one of wildcat_dtype */
  WILDCAT_ERR_SHAPE = -3,      /* sizes out of range (see the descriptors) */
  WILDCAT_ERR_WORKSPACE = -4,  /* workspace missing or smaller than required */
  WILDCAT_ERR_RANGE = -5,      /* wildcat_check_range: an exponent bound exceeds WILDCAT_RANGE_LIMIT */
  WILDCAT_ERR_HIP = -6,        /* a kernel launch or a copy failed */
  WILDCAT_ERR_SCRATCH = -7     /* wildcat_decode_noalloc: the call needs more than its static scratch */
} wildcat_status;

/* Largest exponent argument wildcat_check_range accepts.  exp(64) leaves a
 * factor e^24 of float32 headroom for the sums over up to 2^21 keys and for
 * |V| up to e^9. */
#define WILDCAT_RANGE_LIMIT 64.0

typedef enum { WILDCAT_FP32 = 0, WILDCAT_BF16 = 1 } wildcat_dtype;

/* Storage of the RPNys factor (wildcat_select only; all arithmetic is float64
 * either way).  WILDCAT_FACTOR_F32 is the faster selection the pages leave to
 * future work: each new factor column is computed in float64 and rounded once
 * to float32 for storage, the residual diagonal is lowered by the square of
 * the stored value and L holds the stored values.  It halves the bytes a round
 * streams; the draws then follow the float32-stored factor, so they match the
 * float64 mode's only while the decision margins exceed its perturbation. */
typedef enum { WILDCAT_FACTOR_F64 = 0, WILDCAT_FACTOR_F32 = 1 } wildcat_factor;

/* Keys/values of all units.  Ranges checked by every call:
 *   batch, kv_heads >= 1 and batch * kv_heads <= 65535;  1 <= n <= 2^21;
 *   d in {16, 32, 64, 128};  1 <= r <= min(n, 4096);  beta > 0 and tau > 0,
 *   both finite;  recentre in {0, 1};  dtype a wildcat_dtype (of K and V);
 *   factor a wildcat_factor (0, the float64 factor, when zero-initialised).
 * K, V, Q, K_S and the workspaces must be 16-byte aligned (WILDCAT_ERR_ARG,
 * or WILDCAT_ERR_WORKSPACE for a workspace, otherwise).                  */
typedef struct {
  int32_t batch, kv_heads, n, d;
  int32_t r;          /* requested coreset size */
  double beta;        /* query kernel h(q,k) = exp(beta <q,k>) */
  double tau;         /* RPNys / weight kernel h_tau(k,k') = exp(beta <k,k'> / tau^2); 1 = h */
  int32_t recentre;   /* 1: keys minus their per-unit mean for select and weights */
  int32_t dtype;      /* wildcat_dtype of K and V */
  int32_t factor;     /* wildcat_factor: storage of the RPNys factor */
} wildcat_kv_desc;

/* Queries.  q_heads a positive multiple of kv_heads, batch * q_heads <=
 * 65535; 1 <= m <= 2^24; d, r (<= 4096), beta and dtype as in the kv
 * descriptor used for the compressed cache.                               */
typedef struct {
  int32_t batch, q_heads, kv_heads, m, d, r;
  double beta;
  int32_t dtype;      /* wildcat_dtype of Q and K_S */
} wildcat_q_desc;

/* Host.  Workspace bytes wildcat_select needs for `desc` (0 on a bad desc). */
size_t wildcat_select_workspace_bytes(const wildcat_kv_desc* desc);

/* Host.  Workspace bytes wildcat_weights needs for `desc` (0 on a bad desc). */
size_t wildcat_weights_workspace_bytes(const wildcat_kv_desc* desc);

/*
 * RPNys pivot selection  [WildCat, RPNys / Alg. 1 paragraph].
 * Per unit: the residual diagonal starts at h_tau(k_l, k_l); step i draws
 * s_i = min{ l : C_l > u[i] * T } with C the inclusive prefix sums of the
 * residual diagonal in index order and T its total (the first index with
 * positive residual from the end if rounding leaves none), evaluates
 * g = h_tau(K, k_s) - F[:, :i] F[s, :i]^T, sets column i of the factor to
 * g / sqrt(g_s), and lowers the residual diagonal by its square (zero at s).
 * All of this runs in float64, so the draws are reproducible bit for bit
 * (desc->factor selects float64 or float32 storage of the factor, see
 * wildcat_factor).
 *
 *   K          [U][n][d] dtype, read only.
 *   u          [U][r] float64 uniforms in [0, 1): the randomness, supplied by
 *              the caller (one per step).
 *   S          [U][r] int32 out: pivots in draw order, -1 past r_eff.
 *   r_eff      [U] int32 out: number of pivots drawn (<= r).
 *   L          [U][r][r] float64 out: L[j][k] = F[s_j][k] for k <= j, 0 above
 *              the diagonal and past r_eff; h_tau(K_S, K_S) = L L^T.
 *   workspace  >= wildcat_select_workspace_bytes(desc) bytes, 16-byte
 *              aligned; its contents on entry do not matter.
 */
wildcat_status wildcat_select(const wildcat_kv_desc* desc, const void* K,
                              const double* u, int32_t* S, int32_t* r_eff,
                              double* L, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Nystroem weights and value range  [WildCat, Nystroem paragraph; CompressKV /
 * Alg. 2 paragraph; Lem. 1 paragraph].
 * Per unit: Y = h_tau(K_S, K) [V, 1_n] (one exp-kernel contraction, bf16 or
 * fp32 matrix-core inputs with float32 accumulation), then
 * X = L^{-T} (L^{-1} Y) in float64 (two triangular solves through the pivot
 * block), i.e. X = W [V, 1]: V_S = X[:, :d], w = X[:, d].
 *
 *   K, V        [U][n][d] dtype, read only.   S, r_eff, L: outputs of select.
 *   K_S         [U][r][d] dtype out: raw keys K[s_j] (not recentred), 0 rows
 *               past r_eff.
 *   X           [U][r][d+1] float32 out, 0 rows past r_eff.
 *   vmin, vmax  [U][d] float32 out: column minimum / maximum of V over all n.
 *   workspace   >= wildcat_weights_workspace_bytes(desc) bytes, 16-byte
 *               aligned; contents on entry do not matter.
 */
wildcat_status wildcat_weights(const wildcat_kv_desc* desc, const void* K,
                               const void* V, const int32_t* S,
                               const int32_t* r_eff, const double* L, void* K_S,
                               float* X, float* vmin, float* vmax,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Weighted attention over the compressed cache  [WildCat, plug-in estimator
 * paragraph; Lem. 1 paragraph; WtdAttn / Alg. 3 paragraph].
 * Per query row i of query head h (kv unit as above):
 *   N_i = sum_j exp(beta <q_i, K_S[j]>) X[j, :]       (d+1 numbers)
 *   O[i][c] = fmin(fmax(N_i[c] / N_i[d], vmin[c]), vmax[c])
 * Recentring and tau never reach this call: both cancel in the ratio.
 *
 *   Q           [batch][q_heads][m][d] dtype, read only.
 *   K_S, X, vmin, vmax: outputs of wildcat_weights (r rows per unit).
 *   O           [batch][q_heads][m][d] float32 out.
 */
wildcat_status wildcat_attend(const wildcat_q_desc* desc, const void* Q,
                              const void* K_S, const float* X,
                              const float* vmin, const float* vmax, float* O,
                              hipStream_t stream);

/*
 * Generation over the compressed cache  [WildCat, KV-cache paragraph: the
 * compressed keys and values enter the decoding phase through WtdAttn, and
 * m new tokens cost O(rmd + m^2 d); WtdAttn / Alg. 3; Lem. 1 paragraph].
 * The pages give no formula for this step; the reading taken: new token j
 * joins the weighted attention as one more point of weight 1 and value v_j,
 * seen by the queries of tokens i >= j (causal), and the clip range of query
 * i is the cache's range widened by v_0 .. v_i.  Per query row i of query
 * head h (kv unit as above):
 *   N_i = sum_{l<r} exp(beta <q_i, K_S[l]>) X[l, :]
 *       + sum_{j<=i} exp(beta <q_i, K_new[j]>) [V_new[j], 1]       (d+1 numbers)
 *   lo_i[c] = fmin(vmin[c], V_new[0][c], .., V_new[i][c]), hi_i likewise (fmax)
 *   O[i][c] = fmin(fmax(N_i[c] / N_i[d], lo_i[c]), hi_i[c])
 * desc->m is the number of new tokens and query rows per head; desc->r the
 * rank of the cache.  The kernel exponents are not shifted: the exponent
 * contract of wildcat_check_range covers K_new like the cached keys.
 *
 *   Q           [batch][q_heads][m][d] dtype, read only: query row i is the
 *               query of new token i.
 *   K_S, X, vmin, vmax: the cache, as for wildcat_attend (r rows per unit).
 *   K_new, V_new [batch][kv_heads][m][d] dtype, read only: the new tokens'
 *               keys and values, in token order.
 *   O           [batch][q_heads][m][d] float32 out.
 *   workspace   >= wildcat_decode_workspace_bytes(desc) bytes, 16-byte
 *               aligned; contents on entry do not matter.  Holds the staged
 *               cache-plus-tokens operand and the running ranges, or with
 *               m = 1 (one new token: a form of its own, no staging) the
 *               partial sums of each query head's key ranges.
 */
size_t wildcat_decode_workspace_bytes(const wildcat_q_desc* desc);
wildcat_status wildcat_decode(const wildcat_q_desc* desc, const void* Q,
                              const void* K_S, const float* X,
                              const float* vmin, const float* vmax,
                              const void* K_new, const void* V_new, float* O,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Generation over the compressed cache with no allocation, for callers that
 * cannot allocate device memory or pass a workspace (code under graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and kernels as wildcat_decode, whose workspace is here a
 * static device array of WILDCAT_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU it runs on, held until the process ends; its device address
 * is looked up on the first call on each device).  It calls no allocator.
 * Returns WILDCAT_ERR_SCRATCH, before any launch, when
 * wildcat_decode_workspace_bytes(desc) exceeds that size (e.g. 32 query
 * heads over 8 kv heads, d = 128, r = 1024: up to 1,878 new tokens per call;
 * one new token needs 130 KB), and the status codes of wildcat_decode
 * otherwise (an invalid descriptor: WILDCAT_ERR_ARG or WILDCAT_ERR_SHAPE).
 * Every call on one GPU uses the same scratch: calls that overlap in time on
 * one GPU (other streams, other host threads) race and must be serialised by
 * the caller.  Nothing carries over between calls (every scratch byte read is
 * written first in the same call).
 */
#define WILDCAT_NOALLOC_SCRATCH_BYTES (32u << 20)
wildcat_status wildcat_decode_noalloc(const wildcat_q_desc* desc, const void* Q,
                                      const void* K_S, const float* X,
                                      const float* vmin, const float* vmax,
                                      const void* K_new, const void* V_new, float* O,
                                      hipStream_t stream);

/*
 * Binned RPNys  [WildCat, RPNys / Alg. 1 paragraph: the divide-and-conquer
 * strategy with B bins and a coreset of size r/B per bin, O(nr^2/B^2 + nrd/B)
 * operations].  The bins of a unit are B contiguous blocks of n/B keys, each
 * an independent RPNys problem with its own Nystroem weights (block-diagonal
 * W), and the coreset is the bins' coresets in bin order.  Because the bins
 * are contiguous, the bin-major view of the inputs is the same memory:
 *   K, V   [batch][kv_heads * B][n/B][d]     u  [U * B][r/B]
 * so wildcat_select and wildcat_weights run binning unchanged on a descriptor
 * with kv_heads * B heads, n/B keys and rank r/B (S then holds indices local
 * to each bin, r_eff is per bin).  Their outputs K_S [batch][kv_heads*B][r/B][d]
 * and X [..][r/B][d+1] are, as memory, the concatenated per-unit coresets
 * [batch][kv_heads][r][d] and [..][r][d+1] that wildcat_attend takes with
 * rank r.  The one step in between is this call: the value range that attend
 * clips to is over all n rows of the unit, i.e. the min / max over its bins.
 *
 *   units       batch * kv_heads;  bins >= 1, units * bins <= 65535;
 *               d in {16, 32, 64, 128}.
 *   vmin_bins, vmax_bins  [units * bins][d] float32 (wildcat_weights on the
 *               bin-major view), read only.
 *   vmin, vmax  [units][d] float32 out.
 */
wildcat_status wildcat_merge_value_ranges(int32_t units, int32_t bins, int32_t d,
                                          const float* vmin_bins, const float* vmax_bins,
                                          float* vmin, float* vmax, hipStream_t stream);

/*
 * Input-range guard  [WildCat: the exponential kernel h(q, k) = exp(beta
 * <q, k>) of the problem statement, used here without a stabilising shift].
 * Bounds every exponent argument the three calls can meet, by Cauchy-Schwarz:
 *   E_k = beta / tau^2 * max_l |k_l|^2      (x4 with recentring:
 *                                            |k - kbar| <= 2 max |k|)
 *   E_q = beta * max_i |q_i| * max_l |k_l|  (only if qdesc and Q are given)
 * over all units, with the squared norms summed in float64 on the GPU.
 * HOST-SYNCHRONOUS: enqueues two small reductions on `stream`, copies two
 * doubles back and synchronises `stream` before returning.  Not for capture
 * into a graph.  Returns WILDCAT_ERR_RANGE if E_k or E_q exceeds
 * WILDCAT_RANGE_LIMIT or is not finite (a NaN or inf input counts as inf).
 *
 *   desc, K     as for wildcat_select (K read only).
 *   qdesc, Q    as for wildcat_attend, or both NULL; qdesc->d and
 *               qdesc->dtype must equal desc->d and desc->dtype.
 *   scratch     device, >= 2 doubles, 8-byte aligned; overwritten.
 *   bounds      host, 2 doubles out (may be NULL): {E_k, E_q} (E_q = 0
 *               without queries); written whenever the reductions ran.
 * Argument problems return WILDCAT_ERR_ARG / _DTYPE / _SHAPE before any
 * launch; WILDCAT_ERR_HIP if a launch, the copy or the synchronisation
 * failed.
 */
wildcat_status wildcat_check_range(const wildcat_kv_desc* desc, const void* K,
                                   const wildcat_q_desc* qdesc, const void* Q,
                                   double* scratch, double* bounds,
                                   hipStream_t stream);

/* Host.  Static description of a status code (a wildcat_status value; any
 * other int gives "unknown status"). */
const char* wildcat_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* WILDCAT_H */
