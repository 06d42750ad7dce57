// C ABI of liblrmoe: host-side argument checks, workspace sizing and dispatch to the
// kernels of each step. Every check runs before any launch; nothing here allocates,
// synchronises or keeps state.
#include <algorithm>
#include <vector>

#include "common.h"

using namespace lrmoe;

namespace {

lrmoe_status check_problem(const lrmoe_problem* p, int64_t* K_tot, std::vector<int64_t>* cseg) {
  if (!p || !p->seg_off || !p->quota) return LRMOE_ERR_INVALID_ARG;
  if (p->reserved != 0) return LRMOE_ERR_INVALID_ARG;
  if (p->E < 1 || p->E > 65535 || p->T < 0 || p->K < 1 || p->N < 0) return LRMOE_ERR_INVALID_ARG;
  if (p->D < 8 || p->F < 8) return LRMOE_ERR_INVALID_ARG;
  if (p->dtype != LRMOE_F32 && p->dtype != LRMOE_BF16) return LRMOE_ERR_UNSUPPORTED;
  if (p->swiglu != 0 && p->swiglu != 1) return LRMOE_ERR_INVALID_ARG;
  if (p->D % 8 != 0 || p->F % 8 != 0) return LRMOE_ERR_UNSUPPORTED;
  if ((int64_t)p->T * p->K >= ((int64_t)1 << 31)) return LRMOE_ERR_UNSUPPORTED;
  if (p->seg_off[0] != 0 || p->seg_off[p->E] != p->N) return LRMOE_ERR_INVALID_ARG;
  if (p->N > (int64_t)p->T * p->K) return LRMOE_ERR_INVALID_ARG;  // each (token, slot) holds one pair
  for (int e = 0; e < p->E; ++e)
    if (p->seg_off[e + 1] < p->seg_off[e]) return LRMOE_ERR_INVALID_ARG;
  int64_t k = 0;
  if (cseg) cseg->assign(p->E + 1, 0);
  for (int e = 0; e < p->E; ++e) {
    const int64_t n = p->seg_off[e + 1] - p->seg_off[e];
    const int64_t q = p->quota[e];
    if (q < 0 || q > n) return LRMOE_ERR_INFEASIBLE_QUOTA;
    k += q;
    if (cseg) (*cseg)[e + 1] = k;
  }
  if (K_tot) *K_tot = k;
  return LRMOE_OK;
}

size_t ws_need(const lrmoe_problem* p, lrmoe_compact_mode mode) {
  std::vector<int64_t> cseg;
  check_problem(p, nullptr, &cseg);
  const int64_t* row_off = mode == LRMOE_COMPACT_ZERO_MASKED ? p->seg_off : cseg.data();
  size_t b = align_up(sizeof(double) * (size_t)p->T, 256);  // score: token norms
  b = std::max(b, select_ws_bytes(p));
  b = std::max(b, compact_ws_bytes(p));
  b = std::max(b, gemm_ws_bytes(p, row_off));
  b = std::max(b, scatter_ws_bytes(p));
  return std::max<size_t>(b, 256);
}

// Buffers of one physical-compaction backward at K_tot retained pairs (the list is in the
// header, with lrmoe_backward_bytes); the workspace is added by backward_estimate.
size_t backward_buffer_bytes(const lrmoe_problem* p, int64_t K_tot, bool packed) {
  const size_t e = p->dtype == LRMOE_BF16 ? 2 : 4, K = (size_t)K_tot, N = (size_t)p->N;
  const size_t D = (size_t)p->D, F = (size_t)p->F, E = (size_t)p->E, T = (size_t)p->T;
  const bool sw = p->swiglu != 0;
  const size_t w = sw ? D : F;
  size_t b = N * sizeof(float) + N;            // R, keep
  b += K * 3 * sizeof(int32_t);                // sel, ctok, cslot
  if (!packed) b += K * F * e;                 // PhiW
  else b += K * D * e + K * F * e + (sw ? K * D * e + K * 2 * F * e : 0);  // Dlt, PhiC (XC, HC)
  if (sw) b += K * 2 * F * e;                  // dH
  b += K * w * e;                              // dIn
  b += E * F * D * sizeof(float);              // dW2
  if (sw) b += E * D * 2 * F * sizeof(float);  // dW1
  b += T * w * sizeof(float);                  // scatter output
  return b;
}

// The admission estimate at p's quotas: the backward's buffers plus the library's scratch
// at those quotas: the workspace (physical compaction) and the (token, slot) -> packed row
// map int32 [T x K] that the selection writes for compaction and the scatter.
size_t backward_estimate(const lrmoe_problem* p, int64_t K_tot, bool packed) {
  return backward_buffer_bytes(p, K_tot, packed) + ws_need(p, LRMOE_COMPACT_PHYSICAL) +
         sizeof(int32_t) * (size_t)p->T * p->K;
}

#define LRMOE_TRY(x)                      \
  do {                                    \
    const lrmoe_status st_ = (x);         \
    if (st_ != LRMOE_OK) return st_;      \
  } while (0)

}  // namespace

extern "C" {

const char* lrmoe_status_string(lrmoe_status s) {
  switch (s) {
    case LRMOE_OK: return "ok";
    case LRMOE_ERR_INVALID_ARG: return "invalid argument";
    case LRMOE_ERR_INFEASIBLE_QUOTA: return "infeasible quota (need 0 <= q_e <= n_e)";
    case LRMOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LRMOE_ERR_WORKSPACE: return "workspace missing or too small";
    case LRMOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* lrmoe_version(void) { return "lrmoe 0.1 gfx950"; }

lrmoe_status lrmoe_validate(const lrmoe_problem* p, int64_t* K_tot, int64_t* cseg_off) {
  std::vector<int64_t> cseg;
  int64_t k = 0;
  LRMOE_TRY(check_problem(p, &k, &cseg));
  if (K_tot) *K_tot = k;
  if (cseg_off) std::copy(cseg.begin(), cseg.end(), cseg_off);
  return LRMOE_OK;
}

lrmoe_status lrmoe_backward_bytes(const lrmoe_problem* p, int32_t packed, size_t* bytes) {
  if (!bytes) return LRMOE_ERR_INVALID_ARG;
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, nullptr));
  *bytes = backward_estimate(p, K_tot, packed != 0);
  return LRMOE_OK;
}

lrmoe_status lrmoe_plan_quotas(const lrmoe_problem* p, const int32_t* rho_num, const int32_t* rho_den,
                               int32_t n_rho, int32_t packed, size_t hbm_avail, int32_t* chosen,
                               int32_t* quota_out, size_t* bytes) {
  if (!p || !rho_num || !rho_den || n_rho < 1 || !chosen || !quota_out || !bytes) return LRMOE_ERR_INVALID_ARG;
  *chosen = -1;
  for (int i = 0; i < n_rho; ++i)
    if (rho_den[i] <= 0 || rho_num[i] < 0 || rho_num[i] > rho_den[i]) return LRMOE_ERR_INVALID_ARG;
  if (p->E < 1 || p->E > 65535 || !p->seg_off) return LRMOE_ERR_INVALID_ARG;
  // the problem is checked with all-zero quotas (always feasible) for everything but them
  std::vector<int32_t> q(p->E, 0);
  lrmoe_problem pq = *p;
  pq.quota = q.data();
  LRMOE_TRY(check_problem(&pq, nullptr, nullptr));
  std::vector<int> order(n_rho);
  for (int i = 0; i < n_rho; ++i) order[i] = i;
  // decreasing ratio, equal ratios in index order: a/b > c/d  <=>  a*d > c*b (positive b, d)
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return (int64_t)rho_num[a] * rho_den[b] > (int64_t)rho_num[b] * rho_den[a];
  });
  for (int i : order) {
    int64_t K_tot = 0;
    for (int e = 0; e < p->E; ++e) {
      const int64_t n = p->seg_off[e + 1] - p->seg_off[e];
      const int64_t c = (n * rho_num[i] + rho_den[i] - 1) / rho_den[i];  // ceil(rho n), n >= 0
      q[e] = (int32_t)std::min(n, c);
      K_tot += q[e];
    }
    const size_t b = backward_estimate(&pq, K_tot, packed != 0);  // pq.quota points at q
    if (b <= hbm_avail) {
      *chosen = i;
      std::copy(q.begin(), q.end(), quota_out);
      *bytes = b;
      return LRMOE_OK;
    }
  }
  return LRMOE_ERR_INFEASIBLE_QUOTA;
}

lrmoe_status lrmoe_workspace_size(const lrmoe_problem* p, lrmoe_compact_mode mode, size_t* bytes) {
  if (!bytes) return LRMOE_ERR_INVALID_ARG;
  if (mode != LRMOE_COMPACT_PHYSICAL && mode != LRMOE_COMPACT_ZERO_MASKED) return LRMOE_ERR_INVALID_ARG;
  LRMOE_TRY(check_problem(p, nullptr, nullptr));
  *bytes = ws_need(p, mode);
  return LRMOE_OK;
}

lrmoe_status lrmoe_score(const lrmoe_problem* p, const void* G, const void* Phi, const float* alpha,
                         const int32_t* tok, float* R, void* ws, size_t ws_bytes, lrmoe_stream_t stream) {
  LRMOE_TRY(check_problem(p, nullptr, nullptr));
  if ((p->T > 0 && !G) || (p->N > 0 && (!Phi || !alpha || !tok || !R))) return LRMOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < align_up(sizeof(double) * (size_t)p->T, 256)) return LRMOE_ERR_WORKSPACE;
  return launch_score(p, G, Phi, alpha, tok, R, (double*)ws, (hipStream_t)stream);
}

lrmoe_status lrmoe_score_criterion(const lrmoe_problem* p, lrmoe_criterion criterion, const void* G,
                                   const void* Phi, const float* alpha, const int32_t* tok, float* R, void* ws,
                                   size_t ws_bytes, lrmoe_stream_t stream) {
  if (criterion == LRMOE_CRITERION_LRM) return lrmoe_score(p, G, Phi, alpha, tok, R, ws, ws_bytes, stream);
  if (criterion != LRMOE_CRITERION_GRAD_SQNORM && criterion != LRMOE_CRITERION_GRAD_ABS)
    return LRMOE_ERR_INVALID_ARG;
  LRMOE_TRY(check_problem(p, nullptr, nullptr));
  if ((p->T > 0 && !G) || (p->N > 0 && (!tok || !R))) return LRMOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < align_up(sizeof(double) * (size_t)p->T, 256)) return LRMOE_ERR_WORKSPACE;
  return launch_score_gradient(p, criterion == LRMOE_CRITERION_GRAD_ABS, G, tok, R, (double*)ws,
                               (hipStream_t)stream);
}

lrmoe_status lrmoe_expert_forward(const lrmoe_problem* p, const int64_t* seg_off_d, const void* X,
                                  const int32_t* tok, const float* alpha, const void* W1, const void* W2,
                                  void* H, void* Phi, void* Y, lrmoe_stream_t stream) {
  LRMOE_TRY(check_problem(p, nullptr, nullptr));
  if (p->dtype != LRMOE_BF16 || p->swiglu != 1) return LRMOE_ERR_UNSUPPORTED;
  if (p->N == 0) return LRMOE_OK;
  if (!seg_off_d || !X || !tok || !alpha || !W1 || !W2 || !H || !Phi || !Y) return LRMOE_ERR_INVALID_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)p->T * p->D * 2 >= lim || (int64_t)p->D * 2 * p->F * 2 >= lim || (int64_t)p->F * p->D * 2 >= lim)
    return LRMOE_ERR_UNSUPPORTED;
  return launch_expert_forward(p, seg_off_d, X, tok, alpha, W1, W2, H, Phi, Y, (hipStream_t)stream);
}

lrmoe_status lrmoe_select(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                          const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel, uint8_t* keep,
                          const int32_t* tok, const int32_t* slot, int32_t* pmap, int32_t* ctok, int32_t* cslot,
                          void* ws, size_t ws_bytes, lrmoe_stream_t stream) {
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, nullptr));
  if (!seg_off_d || !quota_d || !cseg_off_d) return LRMOE_ERR_INVALID_ARG;
  if ((p->N > 0 && !R) || (K_tot > 0 && !sel)) return LRMOE_ERR_INVALID_ARG;
  if (pmap && ((p->N > 0 && (!tok || !slot)) || (K_tot > 0 && (!ctok || !cslot)))) return LRMOE_ERR_INVALID_ARG;
  if (!pmap && (ctok || cslot)) return LRMOE_ERR_INVALID_ARG;
  if (select_ws_bytes(p) > 0 && (!ws || ws_bytes < select_ws_bytes(p))) return LRMOE_ERR_WORKSPACE;
  return launch_select(p, R, seg_off_d, quota_d, cseg_off_d, sel, keep, tok, slot, pmap, ctok, cslot, ws,
                       (hipStream_t)stream);
}

lrmoe_status lrmoe_select_noalloc(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                                  const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel, uint8_t* keep,
                                  const int32_t* tok, const int32_t* slot, int32_t* pmap, int32_t* ctok,
                                  int32_t* cslot, lrmoe_stream_t stream) {
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, nullptr));
  if (!seg_off_d || !quota_d || !cseg_off_d) return LRMOE_ERR_INVALID_ARG;
  if ((p->N > 0 && !R) || (K_tot > 0 && !sel)) return LRMOE_ERR_INVALID_ARG;
  if (pmap && ((p->N > 0 && (!tok || !slot)) || (K_tot > 0 && (!ctok || !cslot)))) return LRMOE_ERR_INVALID_ARG;
  if (!pmap && (ctok || cslot)) return LRMOE_ERR_INVALID_ARG;
  if (select_ws_bytes(p) > select_noalloc_max_bytes()) return LRMOE_ERR_WORKSPACE;
  return launch_select_noalloc(p, R, seg_off_d, quota_d, cseg_off_d, sel, keep, tok, slot, pmap, ctok, cslot,
                               (hipStream_t)stream);
}

lrmoe_status lrmoe_compact(const lrmoe_problem* p, lrmoe_compact_mode mode, const int32_t* sel,
                           const uint8_t* keep, const void* G, const void* Phi, const void* X, const void* H,
                           const float* alpha, const int32_t* tok, const int32_t* slot, void* Dlt, void* PhiC,
                           void* XC, void* HC, int32_t* ctok, int32_t* cslot, const int32_t* pmap, void* ws,
                           size_t ws_bytes, lrmoe_stream_t stream) {
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, nullptr));
  const bool sw = p->swiglu != 0;
  if (mode == LRMOE_COMPACT_PHYSICAL) {
    if (K_tot == 0) return LRMOE_OK;
    if (!sel || !G || !alpha || !Dlt || !ctok || (PhiC && !Phi)) return LRMOE_ERR_INVALID_ARG;
    if (!pmap && (!tok || !slot || !cslot)) return LRMOE_ERR_INVALID_ARG;
    if (sw && ((XC && !X) || (HC && !H))) return LRMOE_ERR_INVALID_ARG;
    if (!sw && (X || H || XC || HC)) return LRMOE_ERR_INVALID_ARG;
    if (!pmap && (!ws || ws_bytes < compact_ws_bytes(p))) return LRMOE_ERR_WORKSPACE;
    return launch_compact(p, K_tot, false, sel, nullptr, G, Phi, X, H, alpha, tok, slot, Dlt, PhiC, XC, HC,
                          ctok, cslot, pmap, ws, (hipStream_t)stream);
  }
  if (mode == LRMOE_COMPACT_ZERO_MASKED) {
    if (p->N == 0) return LRMOE_OK;
    if (!keep || !G || !alpha || !tok || !Dlt || PhiC || HC || pmap) return LRMOE_ERR_INVALID_ARG;
    if ((ctok || cslot) && !slot) return LRMOE_ERR_INVALID_ARG;
    if (sw && XC && !X) return LRMOE_ERR_INVALID_ARG;
    if (!sw && (X || XC)) return LRMOE_ERR_INVALID_ARG;
    return launch_compact(p, p->N, true, nullptr, keep, G, Phi, X, H, alpha, tok, slot, Dlt, nullptr, XC,
                          nullptr, ctok, cslot, nullptr, nullptr, (hipStream_t)stream);
  }
  return LRMOE_ERR_INVALID_ARG;
}

lrmoe_status lrmoe_grouped_gemm_bwd(const lrmoe_problem* p, lrmoe_compact_mode mode, const int64_t* row_off_d,
                                    const void* Dlt, const void* PhiC, const void* XC, const void* HC,
                                    const int32_t* hc_rows, const int32_t* phi_rows, const int32_t* x_rows,
                                    const void* W2, const void* W1, float* dW2, float* dW1, void* dH, void* dIn,
                                    int32_t accumulate, void* ws, size_t ws_bytes, lrmoe_stream_t stream,
                                    lrmoe_event_t din_ready) {
  std::vector<int64_t> cseg;
  LRMOE_TRY(check_problem(p, nullptr, &cseg));
  if (mode != LRMOE_COMPACT_PHYSICAL && mode != LRMOE_COMPACT_ZERO_MASKED) return LRMOE_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return LRMOE_ERR_INVALID_ARG;
  const int64_t* row_off_h = mode == LRMOE_COMPACT_ZERO_MASKED ? p->seg_off : cseg.data();
  const int64_t rows = row_off_h[p->E];
  if (!row_off_d || !W2 || !dW2) return LRMOE_ERR_INVALID_ARG;
  if (rows > 0 && (!Dlt || !PhiC || !dIn)) return LRMOE_ERR_INVALID_ARG;
  if (p->swiglu) {
    if (!W1 || !dW1 || (rows > 0 && (!XC || !HC || !dH))) return LRMOE_ERR_INVALID_ARG;
  } else if (W1 || dW1 || dH || XC || HC || hc_rows || x_rows) {
    return LRMOE_ERR_INVALID_ARG;
  }
  // the gathering loads address a gathered matrix with 32-bit byte offsets
  const int64_t esz = p->dtype == LRMOE_BF16 ? 2 : 4, kLim = (int64_t)1 << 31;
  if ((phi_rows && p->N * p->F * esz >= kLim) || (x_rows && (int64_t)p->T * p->D * esz >= kLim))
    return LRMOE_ERR_UNSUPPORTED;
  if (ws_bytes < gemm_ws_bytes(p, row_off_h) || (!ws && gemm_ws_bytes(p, row_off_h) > 0))
    return LRMOE_ERR_WORKSPACE;
  return launch_grouped_gemm_bwd(p, row_off_h, row_off_d, Dlt, PhiC, XC, HC, hc_rows, phi_rows, x_rows, nullptr,
                                 nullptr, W2, W1, dW2, dW1, dH, dIn, accumulate, ws, (hipStream_t)stream,
                                 (hipEvent_t)din_ready);
}

lrmoe_status lrmoe_compact_weighted(const lrmoe_problem* p, const int32_t* sel, const void* Phi, const float* alpha,
                                    void* PhiW, lrmoe_stream_t stream) {
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, nullptr));
  if (K_tot == 0) return LRMOE_OK;
  if (!sel || !Phi || !alpha || !PhiW) return LRMOE_ERR_INVALID_ARG;
  return launch_compact_weighted_phi(p, K_tot, sel, Phi, alpha, PhiW, (hipStream_t)stream);
}

lrmoe_status lrmoe_grouped_gemm_bwd_gathered(const lrmoe_problem* p, const int64_t* cseg_off_d, const void* G,
                                             const float* alpha, const int32_t* sel, const int32_t* ctok,
                                             const void* PhiW, const void* X, const void* H, const void* W2,
                                             const void* W1, float* dW2, float* dW1, void* dH, void* dIn,
                                             int32_t accumulate, void* ws, size_t ws_bytes, lrmoe_stream_t stream,
                                             lrmoe_event_t din_ready) {
  std::vector<int64_t> cseg;
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, &cseg));
  if (accumulate != 0 && accumulate != 1) return LRMOE_ERR_INVALID_ARG;
  if (!cseg_off_d || !W2 || !dW2) return LRMOE_ERR_INVALID_ARG;
  if (K_tot > 0 && (!G || !alpha || !sel || !ctok || !PhiW || !dIn)) return LRMOE_ERR_INVALID_ARG;
  if (p->swiglu) {
    if (!W1 || !dW1 || (K_tot > 0 && (!X || !H || !dH))) return LRMOE_ERR_INVALID_ARG;
  } else if (W1 || dW1 || dH || X || H) {
    return LRMOE_ERR_INVALID_ARG;
  }
  // G and X are read by token with 32-bit byte offsets
  const int64_t esz = p->dtype == LRMOE_BF16 ? 2 : 4;
  if ((int64_t)p->T * p->D * esz >= ((int64_t)1 << 31)) return LRMOE_ERR_UNSUPPORTED;
  const size_t need = gemm_ws_bytes(p, cseg.data());
  if (ws_bytes < need || (!ws && need > 0)) return LRMOE_ERR_WORKSPACE;
  return launch_grouped_gemm_bwd(p, cseg.data(), cseg_off_d, G, PhiW, X, H, sel, nullptr, p->swiglu ? ctok : nullptr,
                                 ctok, alpha, W2, W1, dW2, dW1, dH, dIn, accumulate, ws, (hipStream_t)stream,
                                 (hipEvent_t)din_ready);
}

lrmoe_status lrmoe_scatter(const lrmoe_problem* p, lrmoe_scatter_mode mode, int64_t n_rows, int32_t width,
                           int32_t rows_dtype, const void* rows, const int32_t* ctok, const int32_t* cslot,
                           const int32_t* pmap, float* out, void* ws, size_t ws_bytes, lrmoe_stream_t stream) {
  int64_t K_tot = 0;
  LRMOE_TRY(check_problem(p, &K_tot, nullptr));
  if (mode != LRMOE_SCATTER_TOKEN && mode != LRMOE_SCATTER_SLOT && mode != LRMOE_SCATTER_TOKEN_BESIDE)
    return LRMOE_ERR_INVALID_ARG;
  if (rows_dtype != LRMOE_F32 && rows_dtype != LRMOE_BF16) return LRMOE_ERR_UNSUPPORTED;
  if (n_rows < 0 || n_rows > p->N || width < 8 || width % 8 != 0) return LRMOE_ERR_INVALID_ARG;
  if (!out || (n_rows > 0 && !rows)) return LRMOE_ERR_INVALID_ARG;
  if (pmap) {  // the selection's map addresses the K_tot packed rows
    if (n_rows != K_tot) return LRMOE_ERR_INVALID_ARG;
  } else {
    if (n_rows > 0 && (!ctok || !cslot)) return LRMOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < scatter_ws_bytes(p)) return LRMOE_ERR_WORKSPACE;
  }
  return launch_scatter(p, mode, n_rows, width, rows_dtype, rows, ctok, cslot, pmap, out, ws, (hipStream_t)stream);
}

}  // extern "C"
