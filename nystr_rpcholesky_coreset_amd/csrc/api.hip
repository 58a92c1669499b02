// C ABI of libwildcat.so: argument validation, workspace sizing, dispatch.
// The declarations, with the meaning of every argument, are in wildcat.h.
#include <math.h>

#include "../../include/wildcat.h"
#include "weights_layout.hpp"

namespace wc {
hipError_t launch_select(int bf16, int U, int n, int d, int r, double c, int recentre, int f32_factor, const void* K,
                         const double* u, int32_t* S, int32_t* r_eff, double* L, void* ws, hipStream_t st);
hipError_t launch_weights(int bf16, int U, int n, int d, int r, double c, int recentre, const void* K,
                          const void* V, const int32_t* S, const int32_t* r_eff, const double* L, void* K_S,
                          float* X, float* vmin, float* vmax, void* ws, hipStream_t st);
hipError_t launch_attend(int bf16, int Uq, int group, int m, int d, int r, double beta, const void* Q,
                         const void* K_S, const float* X, const float* vmin, const float* vmax, float* O,
                         hipStream_t st);
hipError_t launch_decode(int bf16, int Uq, int group, int m, int d, int r, double beta, const void* Q,
                         const void* K_S, const float* X, const float* vmin, const float* vmax, const void* Kn,
                         const void* Vn, float* O, void* ws, hipStream_t st);
hipError_t range_norms(int bf16, int d, const void* K, size_t krows, const void* Q, size_t qrows, double* scratch,
                       double (&maxsq)[2], hipStream_t st);
hipError_t launch_merge_ranges(int units, int bins, int d, const float* vmin_b, const float* vmax_b, float* vmin,
                               float* vmax, hipStream_t st);
}  // namespace wc

namespace {

bool valid_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

wildcat_status check_q(const wildcat_q_desc* q) {
  if (q == nullptr) return WILDCAT_ERR_ARG;
  if (q->dtype != WILDCAT_FP32 && q->dtype != WILDCAT_BF16) return WILDCAT_ERR_DTYPE;
  if (!(isfinite(q->beta) && q->beta > 0.0)) return WILDCAT_ERR_ARG;
  if (q->batch < 1 || q->kv_heads < 1 || q->q_heads < 1 || q->q_heads % q->kv_heads != 0 ||
      q->m < 1 || q->m > (1 << 24) || !valid_d(q->d) || q->r < 1 || q->r > wc::kMaxR ||
      (int64_t)q->batch * q->q_heads > 65535)
    return WILDCAT_ERR_SHAPE;
  return WILDCAT_OK;
}

wildcat_status check_kv(const wildcat_kv_desc* k) {
  if (k == nullptr) return WILDCAT_ERR_ARG;
  if (k->dtype != WILDCAT_FP32 && k->dtype != WILDCAT_BF16) return WILDCAT_ERR_DTYPE;
  if (!(isfinite(k->beta) && k->beta > 0.0) || !(isfinite(k->tau) && k->tau > 0.0)) return WILDCAT_ERR_ARG;
  if (k->recentre != 0 && k->recentre != 1) return WILDCAT_ERR_ARG;
  if (k->factor != WILDCAT_FACTOR_F64 && k->factor != WILDCAT_FACTOR_F32) return WILDCAT_ERR_ARG;
  if (k->batch < 1 || k->kv_heads < 1 || k->n < 1 || k->n > wc::kMaxN || !valid_d(k->d)) return WILDCAT_ERR_SHAPE;
  if (k->r < 1 || k->r > k->n || k->r > wc::kMaxR) return WILDCAT_ERR_SHAPE;
  if ((int64_t)k->batch * k->kv_heads > 65535) return WILDCAT_ERR_SHAPE;
  return WILDCAT_OK;
}

}  // namespace

extern "C" {

size_t wildcat_select_workspace_bytes(const wildcat_kv_desc* desc) {
  if (check_kv(desc) != WILDCAT_OK) return 0;
  return wc::SelectLayout(desc->batch * desc->kv_heads, desc->n, desc->d, desc->r,
                          desc->factor == WILDCAT_FACTOR_F32 ? 4 : 8).total;
}

size_t wildcat_weights_workspace_bytes(const wildcat_kv_desc* desc) {
  if (check_kv(desc) != WILDCAT_OK) return 0;
  return wc::WeightsLayout(desc->batch * desc->kv_heads, desc->n, desc->d, desc->r, desc->dtype == WILDCAT_BF16).total;
}

wildcat_status wildcat_select(const wildcat_kv_desc* desc, const void* K, const double* u, int32_t* S,
                              int32_t* r_eff, double* L, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  wildcat_status st = check_kv(desc);
  if (st != WILDCAT_OK) return st;
  if (!K || !u || !S || !r_eff || !L || !aligned16(K)) return WILDCAT_ERR_ARG;
  if (!workspace || !aligned16(workspace) || workspace_bytes < wildcat_select_workspace_bytes(desc))
    return WILDCAT_ERR_WORKSPACE;
  const int U = desc->batch * desc->kv_heads;
  const double c = desc->beta / (desc->tau * desc->tau);
  hipError_t e = wc::launch_select(desc->dtype == WILDCAT_BF16, U, desc->n, desc->d, desc->r, c, desc->recentre,
                                   desc->factor == WILDCAT_FACTOR_F32,
                                   K, u, S, r_eff, L, workspace, stream);
  return e == hipSuccess ? WILDCAT_OK : WILDCAT_ERR_HIP;
}

wildcat_status wildcat_weights(const wildcat_kv_desc* desc, const void* K, const void* V, const int32_t* S,
                               const int32_t* r_eff, const double* L, void* K_S, float* X, float* vmin,
                               float* vmax, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  wildcat_status st = check_kv(desc);
  if (st != WILDCAT_OK) return st;
  if (!K || !V || !S || !r_eff || !L || !K_S || !X || !vmin || !vmax) return WILDCAT_ERR_ARG;
  if (!aligned16(K) || !aligned16(V) || !aligned16(K_S)) return WILDCAT_ERR_ARG;
  if (!workspace || !aligned16(workspace) || workspace_bytes < wildcat_weights_workspace_bytes(desc))
    return WILDCAT_ERR_WORKSPACE;
  const int U = desc->batch * desc->kv_heads;
  const double c = desc->beta / (desc->tau * desc->tau);
  hipError_t e = wc::launch_weights(desc->dtype == WILDCAT_BF16, U, desc->n, desc->d, desc->r, c, desc->recentre,
                                    K, V, S, r_eff, L, K_S, X, vmin, vmax, workspace, stream);
  return e == hipSuccess ? WILDCAT_OK : WILDCAT_ERR_HIP;
}

wildcat_status wildcat_attend(const wildcat_q_desc* desc, const void* Q, const void* K_S, const float* X,
                              const float* vmin, const float* vmax, float* O, hipStream_t stream) {
  const wildcat_status qs = check_q(desc);
  if (qs != WILDCAT_OK) return qs;
  if (!Q || !K_S || !X || !vmin || !vmax || !O || !aligned16(Q) || !aligned16(K_S)) return WILDCAT_ERR_ARG;
  const int Uq = desc->batch * desc->q_heads;
  const int group = desc->q_heads / desc->kv_heads;
  hipError_t e = wc::launch_attend(desc->dtype == WILDCAT_BF16, Uq, group, desc->m, desc->d, desc->r, desc->beta,
                                   Q, K_S, X, vmin, vmax, O, stream);
  return e == hipSuccess ? WILDCAT_OK : WILDCAT_ERR_HIP;
}

size_t wildcat_decode_workspace_bytes(const wildcat_q_desc* desc) {
  if (check_q(desc) != WILDCAT_OK) return 0;
  return wc::DecodeLayout(desc->batch * desc->kv_heads, desc->m, desc->d, desc->r, desc->dtype == WILDCAT_BF16,
                          desc->batch * desc->q_heads).total;
}

wildcat_status wildcat_decode(const wildcat_q_desc* desc, const void* Q, const void* K_S, const float* X,
                              const float* vmin, const float* vmax, const void* K_new, const void* V_new, float* O,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const wildcat_status qs = check_q(desc);
  if (qs != WILDCAT_OK) return qs;
  if (!Q || !K_S || !X || !vmin || !vmax || !K_new || !V_new || !O) return WILDCAT_ERR_ARG;
  if (!aligned16(Q) || !aligned16(K_S) || !aligned16(K_new) || !aligned16(V_new)) return WILDCAT_ERR_ARG;
  if (!workspace || !aligned16(workspace) || workspace_bytes < wildcat_decode_workspace_bytes(desc))
    return WILDCAT_ERR_WORKSPACE;
  const int Uq = desc->batch * desc->q_heads;
  const int group = desc->q_heads / desc->kv_heads;
  hipError_t e = wc::launch_decode(desc->dtype == WILDCAT_BF16, Uq, group, desc->m, desc->d, desc->r, desc->beta, Q,
                                   K_S, X, vmin, vmax, K_new, V_new, O, workspace, stream);
  return e == hipSuccess ? WILDCAT_OK : WILDCAT_ERR_HIP;
}

wildcat_status wildcat_check_range(const wildcat_kv_desc* desc, const void* K, const wildcat_q_desc* qdesc,
                                   const void* Q, double* scratch, double* bounds, hipStream_t stream) {
  wildcat_status st = check_kv(desc);
  if (st != WILDCAT_OK) return st;
  if (!K || !aligned16(K) || !scratch || (reinterpret_cast<uintptr_t>(scratch) & 7u) != 0) return WILDCAT_ERR_ARG;
  if ((qdesc == nullptr) != (Q == nullptr)) return WILDCAT_ERR_ARG;
  size_t qrows = 0;
  if (qdesc) {
    if ((st = check_q(qdesc)) != WILDCAT_OK) return st;
    if (!aligned16(Q)) return WILDCAT_ERR_ARG;
    if (qdesc->dtype != desc->dtype) return WILDCAT_ERR_DTYPE;
    if (qdesc->d != desc->d) return WILDCAT_ERR_SHAPE;
    qrows = (size_t)qdesc->batch * qdesc->q_heads * qdesc->m;
  }
  const size_t krows = (size_t)desc->batch * desc->kv_heads * desc->n;
  double maxsq[2];
  const hipError_t e = wc::range_norms(desc->dtype == WILDCAT_BF16, desc->d, K, krows, Q, qrows, scratch, maxsq,
                                       stream);
  if (e != hipSuccess) return WILDCAT_ERR_HIP;
  const double ek = desc->beta / (desc->tau * desc->tau) * maxsq[0] * (desc->recentre ? 4.0 : 1.0);
  const double eq = qdesc ? qdesc->beta * sqrt(maxsq[1]) * sqrt(maxsq[0]) : 0.0;
  if (bounds) {
    bounds[0] = ek;
    bounds[1] = eq;
  }
  if (!(ek <= WILDCAT_RANGE_LIMIT) || !(eq <= WILDCAT_RANGE_LIMIT)) return WILDCAT_ERR_RANGE;
  return WILDCAT_OK;
}

wildcat_status wildcat_merge_value_ranges(int32_t units, int32_t bins, int32_t d, const float* vmin_bins,
                                          const float* vmax_bins, float* vmin, float* vmax, hipStream_t stream) {
  if (units < 1 || bins < 1 || !valid_d(d) || (int64_t)units * bins > 65535) return WILDCAT_ERR_SHAPE;
  if (!vmin_bins || !vmax_bins || !vmin || !vmax) return WILDCAT_ERR_ARG;
  const hipError_t e = wc::launch_merge_ranges(units, bins, d, vmin_bins, vmax_bins, vmin, vmax, stream);
  return e == hipSuccess ? WILDCAT_OK : WILDCAT_ERR_HIP;
}

const char* wildcat_status_string(int status) {
  switch (status) {
    case WILDCAT_OK: return "ok";
    case WILDCAT_ERR_ARG: return "invalid argument (null or misaligned pointer, bad beta/tau/recentre/factor)";
    case WILDCAT_ERR_DTYPE: return "unsupported dtype";
    case WILDCAT_ERR_SHAPE: return "shape out of range";
    case WILDCAT_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case WILDCAT_ERR_RANGE: return "an exponent bound of the inputs exceeds WILDCAT_RANGE_LIMIT (or is not finite)";
    case WILDCAT_ERR_HIP: return "HIP launch failed";
    case WILDCAT_ERR_SCRATCH: return "the call needs more than the static scratch of the no-allocation entry point";
  }
  return "unknown status";
}

}  // extern "C"
