/*
 * lrmoe.h - C ABI of the memory-aware MoE expert backward on one MI355X (gfx950).
 *
 * The library implements the backward-time calibration of the LRMoE paper
 * ("LRMoE: Demand-Side Load Re-Calibration for Efficient MoE Training on
 * Memory-Constrained Nodes"): its Algorithm 1 (section 3.3) scores every routed
 * token-expert pair, keeps a fixed per-expert quota of the best pairs, packs the
 * retained rows, runs the expert backward on the packed rows and maps the input
 * gradients back. One call per step:
 *
 *   lrmoe_score            LRM score of every pair           (section 3.2, Eq. 3)
 *   lrmoe_select           per-expert top-q under quotas      (section 3.3; appendix 7.2)
 *   lrmoe_compact          packing into expert segments       (sections 3.1, 3.4, Figure 4)
 *   lrmoe_grouped_gemm_bwd variable-size grouped GEMMs        (section 3.4)
 *   or, with the gradient rows read by token instead of packed:
 *   lrmoe_compact_weighted, lrmoe_grouped_gemm_bwd_gathered
 *   lrmoe_scatter          inverse mapping to token order     (section 3.1)
 *
 * Beside the path:
 *
 *   lrmoe_score_criterion  the ablation's gradient-only scores (section 4.7, Table 2)
 *   lrmoe_expert_forward   the forward that saves the backward's context
 *                          (Algorithm 1, FullForwardAndSaveContext)
 *   lrmoe_backward_bytes,  host-only: the device bytes a backward holds, and quota
 *   lrmoe_plan_quotas      admission on one GPU (Algorithm 1's admission, section 3.3)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pairs are stored expert-major: expert e owns pair rows [seg_off[e], seg_off[e+1]).
 * - Packed ("compact") rows are expert-major too: expert e owns packed rows
 *   [cseg_off[e], cseg_off[e+1]) with cseg_off = exclusive prefix sum of the quotas.
 *   Inside a segment the retained pairs keep their ascending original order.
 * - Expert weights are stored [in x out], row-major: W2[e] is [F x D] (FC2, the
 *   protected projection whose input is phi), W1[e] is [D x 2F] (FC1) whose columns
 *   [0,F) are the gate and [F,2F) the up projection of a SwiGLU expert,
 *   phi = silu(gate) * up.
 * - "storage dtype" (problem.dtype) is the dtype of G, Phi, X, H, W1, W2 and of the
 *   packed and gradient rows (Dlt, PhiC, XC, HC, dH, dIn). bf16 tensors hold raw
 *   bf16 bit patterns. Weight gradients dW1/dW2, scores and scatter outputs are f32.
 * - All pointers other than those documented "host" are device pointers. Row-major,
 *   dense, 16-byte aligned; D and F must be multiples of 8.
 * - Ownership: the caller owns every buffer. The library allocates nothing, frees
 *   nothing and keeps no state between calls. Scratch memory comes through the
 *   (ws, ws_bytes) arguments; lrmoe_workspace_size gives the size.
 * - Streams: every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream) and never synchronises it. Argument checks run on the host before any
 *   launch; on error nothing is launched.
 * - Quotas are fixed before the call (section 3.1: quotas remain fixed for the
 *   invocation). A quota outside 0 <= q_e <= n_e is LRMOE_ERR_INFEASIBLE_QUOTA,
 *   the analogue of Algorithm 1's "return Infeasible".
 */
#ifndef LRMOE_H
#define LRMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same types as HIP's hipStream_t and hipEvent_t. */
typedef struct ihipStream_t* lrmoe_stream_t;
typedef struct ihipEvent_t* lrmoe_event_t;

typedef enum lrmoe_status {
  LRMOE_OK = 0,
  LRMOE_ERR_INVALID_ARG = 1,       /* null pointer, bad size, non-monotone offsets ... */
  LRMOE_ERR_INFEASIBLE_QUOTA = 2,  /* some q_e < 0 or q_e > n_e                         */
  LRMOE_ERR_UNSUPPORTED = 3,       /* shape/dtype combination not implemented          */
  LRMOE_ERR_WORKSPACE = 4,         /* ws is NULL or smaller than lrmoe_workspace_size  */
  LRMOE_ERR_HIP = 5                /* a HIP launch failed                              */
} lrmoe_status;

typedef enum lrmoe_dtype { LRMOE_F32 = 0, LRMOE_BF16 = 1 } lrmoe_dtype;

/* PHYSICAL: retained rows are copied into K_tot-row packed buffers (section 3.4).
 * ZERO_MASKED: the same-shape baseline of section 3.4 - N-row buffers in which the
 * dropped pairs' gradient rows are zero; the GEMMs then run over all N rows. */
typedef enum lrmoe_compact_mode { LRMOE_COMPACT_PHYSICAL = 0, LRMOE_COMPACT_ZERO_MASKED = 1 } lrmoe_compact_mode;

/* TOKEN: out[t] = sum of the rows of token t (back to token order).
 * SLOT:  out[t*K + k] = the row of pair (t, k), every other row zero
 *        ((token, routing-slot) positions in a zero-initialised buffer, section 3.1).
 * TOKEN_BESIDE: TOKEN's result, bit for bit, from a launch shaped to run on a second
 *        stream beside the grouped GEMM's weight-gradient launch (after din_ready): at most
 *        one block per compute unit, each looping over tokens, with few enough registers
 *        to share the compute units that launch occupies. Alone on the GPU it is slower
 *        than TOKEN. */
typedef enum lrmoe_scatter_mode {
  LRMOE_SCATTER_TOKEN = 0,
  LRMOE_SCATTER_SLOT = 1,
  LRMOE_SCATTER_TOKEN_BESIDE = 2
} lrmoe_scatter_mode;

/* Selection criterion of lrmoe_score_criterion (section 4.7, Table 2, the ablation). */
typedef enum lrmoe_criterion {
  LRMOE_CRITERION_LRM = 0,          /* the Load Recalibration Metric, as lrmoe_score     */
  LRMOE_CRITERION_GRAD_SQNORM = 1,  /* squared gradient norm  ||G[tok[j]]||^2            */
  LRMOE_CRITERION_GRAD_ABS = 2      /* absolute gradient magnitude  sum_i |G[tok[j], i]| */
} lrmoe_criterion;

typedef struct lrmoe_problem {
  int32_t E;              /* local experts                                          */
  int32_t T;              /* tokens                                                 */
  int32_t K;              /* routing slots per token (top-K)                        */
  int32_t D;              /* hidden size: width of g_t and x_t                      */
  int32_t F;              /* expert intermediate size: width of phi_u               */
  int32_t swiglu;         /* 1: SwiGLU experts (FC1 + FC2); 0: FC2 only             */
  int32_t dtype;          /* lrmoe_dtype: storage dtype                             */
  int32_t reserved;       /* must be 0                                              */
  int64_t N;              /* routed pairs = seg_off[E]                              */
  const int64_t* seg_off; /* host [E+1]: pair segment offsets, seg_off[0] = 0       */
  const int32_t* quota;   /* host [E]: retention quotas q_e, fixed before the call  */
} lrmoe_problem;

const char* lrmoe_status_string(lrmoe_status s);
const char* lrmoe_version(void);

/* Host-only. Checks the problem (sizes, monotone offsets, N = seg_off[E], quotas
 * 0 <= q_e <= n_e, supported dtype/shape) and returns K_tot = sum q_e and, if
 * cseg_off is not NULL, the packed segment offsets (host [E+1]). Launches nothing. */
lrmoe_status lrmoe_validate(const lrmoe_problem* p, int64_t* K_tot, int64_t* cseg_off);

/* Host-only. Bytes of scratch that every entry point below needs for this problem
 * and compact mode (one buffer serves all of them; calls on one stream may share it).
 * It is the largest of: the score's fp64 token norms [T]; the selection's histograms and
 * chunk counts; the (token, slot) -> packed row map int32 [T x K] of compaction and
 * scatter; the grouped GEMM's weight-gradient plan plus its split-K partials, one
 * 256 x 256 fp32 tile per (chunk, weight-gradient tile) of every expert whose rows (the
 * retained rows q_e, or n_e when zero-masked) are cut into more than one chunk. Chunks hold
 * at most 12288 rows, or 8192 or 6144 when the library's schedule model finds that one
 * expert's long chunks would leave the GPU's eight XCDs unevenly loaded (a deterministic
 * function of the row counts). The partials dominate at large quotas, so the size depends
 * on them. */
lrmoe_status lrmoe_workspace_size(const lrmoe_problem* p, lrmoe_compact_mode mode, size_t* bytes);

/* Host-only. Device bytes one physical-compaction backward holds at p's quotas, besides
 * its inputs (G, Phi, X, H, W1, W2, alpha, tok, slot): its scratch, the workspace
 * (lrmoe_workspace_size for LRMOE_COMPACT_PHYSICAL at these quotas) and the (token, slot)
 * map pmap int32 [T x K] of lrmoe_select, plus the buffers
 *   R f32 [N], keep u8 [N]; sel, ctok, cslot int32 [K_tot]; the packed rows of step 3:
 *   with packed = 0 the weighted saved rows PhiW [K_tot x F] of lrmoe_compact_weighted
 *   (the path of lrmoe_grouped_gemm_bwd_gathered), with packed != 0 the weighted
 *   gradient rows Dlt [K_tot x D] and the packed saved rows PhiC [K_tot x F] (SwiGLU: also
 *   XC [K_tot x D] and HC [K_tot x 2F]); SwiGLU: dH [K_tot x 2F]; dIn [K_tot x w]; f32 weight gradients
 *   dW2 [E x F x D] (SwiGLU: dW1 [E x D x 2F]); the scatter output f32 [T x w]
 * (storage dtype where not marked; w = D for SwiGLU experts, F for FC2-only ones). This is
 * the memory the retention quotas decide: the estimate quota admission compares with the
 * available HBM. */
lrmoe_status lrmoe_backward_bytes(const lrmoe_problem* p, int32_t packed, size_t* bytes);

/* Host-only. Quota admission on one GPU: Algorithm 1's forward-time admission (section
 * 3.3) with a single GPU, so no replica plan and no communication window to check. The
 * n_rho candidate ratios rho_i = rho_num[i] / rho_den[i] (0 <= rho_i <= 1, host arrays)
 * are tried in decreasing order (equal ratios in index order); candidate i gives quotas
 * q_e = min(n_e, ceil(rho_i n_e)) (exact integer arithmetic) and its estimate
 * lrmoe_backward_bytes at those quotas. The first candidate whose estimate is at most
 * hbm_avail is admitted: *chosen = i, quota_out [E] (host) = its quotas, *bytes = its
 * estimate. p->quota is not read (may be NULL). If no candidate fits, the result is
 * LRMOE_ERR_INFEASIBLE_QUOTA (Algorithm 1's "return Infeasible") with *chosen = -1. A ratio
 * outside [0,1], a denominator <= 0 or n_rho < 1 is LRMOE_ERR_INVALID_ARG. */
lrmoe_status lrmoe_plan_quotas(const lrmoe_problem* p, const int32_t* rho_num, const int32_t* rho_den,
                               int32_t n_rho, int32_t packed, size_t hbm_avail, int32_t* chosen,
                               int32_t* quota_out, size_t* bytes);

/* Step 1 - LRM score (section 3.2, Proposition 3.1, Eq. 3; Algorithm 1's scoring step):
 *   R[j] = alpha[j]^2 * ||G[tok[j]]||^2 * ||Phi[j]||^2   for every pair j < N.
 * G [T x D] upstream gradient before the routing weight (appendix 7.1, Eq. 4-5),
 * Phi [N x F] saved FC2 input per pair, alpha [N] f32, tok [N] int32 in [0,T).
 * R [N] f32 out. Norms are accumulated in fp64; R is rounded once to f32. */
lrmoe_status lrmoe_score(const lrmoe_problem* p, const void* G, const void* Phi, const float* alpha,
                         const int32_t* tok, float* R, void* ws, size_t ws_bytes, lrmoe_stream_t stream);

/* Step 1 with another selection criterion: the alternatives the LRM score is compared
 * with in the ablation (section 4.7, Table 2). The gradient-only criteria score pair j
 * from its token's upstream gradient row G[tok[j]] alone (no routing weight, no saved
 * activation): the squared norm, or the sum of magnitudes. LRMOE_CRITERION_LRM is exactly
 * lrmoe_score. For the gradient-only criteria Phi and alpha may be NULL; a token outside
 * [0,T) scores 0. Sums in fp64, R rounded once to f32. Workspace as lrmoe_score; an
 * unknown criterion is LRMOE_ERR_INVALID_ARG. The table's random-selection baseline needs
 * no kernel: its scores are random draws, which the caller passes to lrmoe_select. */
lrmoe_status lrmoe_score_criterion(const lrmoe_problem* p, lrmoe_criterion criterion, const void* G,
                                   const void* Phi, const float* alpha, const int32_t* tok, float* R,
                                   void* ws, size_t ws_bytes, lrmoe_stream_t stream);

/* Step 2 - per-expert TopK under fixed quotas (section 3.3; appendix 7.2, Prop. 7.1):
 * inside each segment keep the q_e largest R; among equal R the lower pair index wins.
 * seg_off_d [E+1] int64, quota_d [E] int32, cseg_off_d [E+1] int64 are device copies of
 * the problem's offsets, quotas and validated packed offsets.
 * sel [K_tot] int32 out: retained pair indices, segment by segment, ascending.
 * keep [N] uint8 out (may be NULL): 1 if retained, else 0.
 * pmap [T x K] int32 out (may be NULL; then tok, slot, ctok, cslot may be NULL and ctok,
 * cslot must be): with tok, slot [N] int32 (the pairs' tokens and routing slots), the
 * (token, slot) -> packed row map of the retained pairs, pmap[t*K + k] = c, -1 where the
 * position holds no retained pair; and for every packed row c its token and slot,
 * ctok[c], cslot[c] [K_tot] int32 (both -1 for a pair whose token is outside [0,T) or
 * slot outside [0,K): such a pair has no position). Compaction and the scatter take pmap
 * instead of building it themselves, so a backward builds it once. Each (token, slot)
 * position must hold at most one pair. */
lrmoe_status lrmoe_select(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                          const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel,
                          uint8_t* keep, const int32_t* tok, const int32_t* slot, int32_t* pmap,
                          int32_t* ctok, int32_t* cslot, void* ws, size_t ws_bytes, lrmoe_stream_t stream);

/* lrmoe_select without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments and results as lrmoe_select minus (ws, ws_bytes). Its scratch is a fixed
 * 4 MiB array of the library's, one per GPU, held until the process ends; the call
 * allocates and frees nothing. The stream's device must be the current device. The
 * selection needs E x 20 KB of digit histograms (one per radix pass), E x 64 B of segment
 * state and 16 B per expert per 4096-pair chunk of the longest segment (each part rounded
 * up to 256 B; about 340 KB for 16 experts of up to 200k pairs); a problem that needs more
 * than 4 MiB is refused with LRMOE_ERR_WORKSPACE before any launch. The selection's first
 * launch clears what it accumulates into, so a call does not depend on the previous call's
 * contents.
 * All calls on one GPU share the array: calls that overlap in time on one GPU (other
 * streams, other host threads) race; calls in order on one stream do not. */
lrmoe_status lrmoe_select_noalloc(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                                  const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel,
                                  uint8_t* keep, const int32_t* tok, const int32_t* slot, int32_t* pmap,
                                  int32_t* ctok, int32_t* cslot, lrmoe_stream_t stream);

/* Step 3 - compaction (section 3.1 "compact runtime", section 3.4 / Figure 4).
 * PHYSICAL, for packed row c < K_tot with j = sel[c], t = tok[j]:
 *   Dlt[c]  = alpha[j] * G[t]   (weighted cotangent, Eq. 5; one rounding to the storage dtype,
 *                                bf16 round-to-nearest-even of the exact product)
 *   PhiC[c] = Phi[j];  XC[c] = X[t];  HC[c] = H[j];  ctok[c] = t;  cslot[c] = slot[j]
 *   Dlt, XC [K_tot x D]; PhiC [K_tot x F]; HC [K_tot x 2F]; ctok, cslot [K_tot] int32.
 *   X, H, XC, HC are used only when swiglu = 1 (else pass NULL). keep is ignored.
 *   PhiC, XC and HC are optional (NULL: not written; Phi, X, H may then be NULL): the
 *   grouped GEMM can read the saved rows in place through sel and ctok (its row maps),
 *   which saves the copies.
 *   Each (token, slot) position holds at most one pair (a token routes to an expert through
 *   one slot); the gather runs token by token through a [T x K] position map, so a token's
 *   G and X rows are read from HBM once for all of its retained pairs. pmap: the map and
 *   ctok/cslot written by lrmoe_select for this sel (tok, slot and cslot may then be NULL,
 *   ctok is read, and neither is written; no workspace needed); NULL: the map is built in
 *   ws and ctok, cslot are written here. A retained pair whose tok is outside [0,T) or slot
 *   outside [0,K) has no position: its ctok and cslot are -1 and its packed rows are zero
 *   (Dlt, and PhiC, XC, HC when requested), so it adds nothing to the later steps.
 * ZERO_MASKED, for every pair j < N: Dlt[j] = keep[j] ? alpha[j] * G[tok[j]] : 0 and
 *   XC[j] = X[tok[j]] (swiglu; XC optional, the GEMM can read X through tok); sel is
 *   ignored; PhiC and HC must be NULL (the GEMMs read Phi and H in place); ctok/cslot, if
 *   not NULL, receive copies of tok/slot; pmap must be NULL. ws may be NULL.
 * ws: scratch of at least lrmoe_workspace_size bytes (PHYSICAL without pmap), else
 * LRMOE_ERR_WORKSPACE. */
lrmoe_status lrmoe_compact(const lrmoe_problem* p, lrmoe_compact_mode mode, const int32_t* sel,
                           const uint8_t* keep, const void* G, const void* Phi, const void* X,
                           const void* H, const float* alpha, const int32_t* tok, const int32_t* slot,
                           void* Dlt, void* PhiC, void* XC, void* HC, int32_t* ctok, int32_t* cslot,
                           const int32_t* pmap, void* ws, size_t ws_bytes, lrmoe_stream_t stream);

/* Step 4 - packed expert backward, variable-size grouped GEMMs (section 3.4: the FC2
 * and FC1 data- and weight-gradient GEMMs on the retained rows; section 3.1: the
 * activation backward between them). Rows of expert e: [row_off[e], row_off[e+1]) with
 * row_off = cseg_off (PHYSICAL) or seg_off (ZERO_MASKED); row_off_d is its device copy.
 * In ZERO_MASKED mode pass Phi as PhiC and H as HC.
 *   dW2[e] (+)= PhiC_e^T Dlt_e                        f32 [E x F x D]
 *   dPhi      = Dlt_e W2[e]^T                         (internal)
 *   dH        = [dPhi*up*silu'(gate), dPhi*silu(gate)] storage dtype [rows x 2F], out
 *   dW1[e] (+)= XC_e^T dH_e                           f32 [E x D x 2F]
 *   dIn       = dH_e W1[e]^T                          storage dtype [rows x D]
 * with gate = HC[r, :F], up = HC[r, F:] for packed row c, where r = hc_rows[c] (hc_rows
 * [rows] int32) or r = c when hc_rows is NULL.
 * Row maps (each [rows] int32 or NULL = identity) let the saved activations be read in
 * place instead of packed: row c of PhiC is PhiC[phi_rows[c]], of XC is XC[x_rows[c]], of
 * HC is HC[hc_rows[c]]. A mapped PhiC or HC has N rows (pair rows), a mapped XC has T rows
 * (token rows); a mapped row outside that range reads as zeros. With a mapped PhiC or XC
 * the matrix must be under 2 GiB (else LRMOE_ERR_UNSUPPORTED).
 *   PHYSICAL, in place: PhiC = Phi, phi_rows = sel; XC = X, x_rows = ctok; HC = H,
 *                       hc_rows = sel (compaction then writes only Dlt, ctok, cslot).
 *   PHYSICAL, packed:   the compacted PhiC, XC, HC and NULL maps.
 *   ZERO_MASKED:        PhiC = Phi, HC = H, XC = X with x_rows = tok (or the masked XC).
 * For swiglu = 0 only dW2 and dIn = dPhi [rows x F] are produced (dH, XC, HC, hc_rows,
 * x_rows, W1, dW1 must be NULL).
 * accumulate = 0 overwrites dW1/dW2 (experts with no rows get 0); 1 adds to them.
 * din_ready (may be NULL): an event the caller created; it is recorded on `stream` as soon
 * as dIn is complete, before the weight-gradient launches, so the caller can start the
 * scatter of dIn on another stream while the weight gradients are computed
 * (LRMOE_SCATTER_TOKEN_BESIDE is shaped for that). A failed record returns LRMOE_ERR_HIP.
 * bf16: MFMA with fp32 accumulation. f32: fp32 FMA throughout. */
lrmoe_status lrmoe_grouped_gemm_bwd(const lrmoe_problem* p, lrmoe_compact_mode mode,
                                    const int64_t* row_off_d, const void* Dlt, const void* PhiC,
                                    const void* XC, const void* HC, const int32_t* hc_rows,
                                    const int32_t* phi_rows, const int32_t* x_rows, const void* W2,
                                    const void* W1, float* dW2, float* dW1, void* dH, void* dIn,
                                    int32_t accumulate, void* ws, size_t ws_bytes, lrmoe_stream_t stream,
                                    lrmoe_event_t din_ready);

/* Step 3 for the path that reads gradient rows by token (no Dlt; section 3.1's compact
 * runtime gathers the retained rows, here the saved activation rows carry the weight).
 * PHYSICAL packing only: for packed row c < K_tot of retained pair j = sel[c],
 *   PhiW[c] = alpha[j] * Phi[j]      storage dtype [K_tot x F], out
 * rounded once to the storage dtype (bf16: nearest-even of the exact product). A pair
 * outside [0, N) gives a zero row. The FC2 weight gradient is linear in each of phi and
 * the gradient row (appendix 7.1, Eq. 6-8), so PhiW^T g_tok over an expert's rows equals
 * PhiC^T Dlt. No workspace; nothing to do when K_tot = 0. */
lrmoe_status lrmoe_compact_weighted(const lrmoe_problem* p, const int32_t* sel, const void* Phi, const float* alpha,
                                    void* PhiW, lrmoe_stream_t stream);

/* Step 4 without a materialised Dlt (section 3.4's grouped GEMMs over the packed
 * segments; section 3.1). PHYSICAL rows: expert e owns packed rows [cseg_off[e],
 * cseg_off[e+1]) (cseg_off_d: device copy, int64 [E+1]). Packed row c belongs to pair
 * j = sel[c] of token t = ctok[c] (the selection's outputs); G [T x D] holds the layer's
 * output-gradient rows by token, read in place:
 *   dPhi[c]   = alpha[j] * (G[t] W2[e]^T)              (internal, fp32 before the scale)
 *   dW2[e] (+)= sum_c PhiW[c]^T G[t]                   f32 [E x F x D]
 *   dH, dW1, dIn as in lrmoe_grouped_gemm_bwd with gate, up = H[j] and the FC1 input
 *   X[t] (H [N x 2F] and X [T x D] read in place); dH [K_tot x 2F], dIn [K_tot x D]
 * PhiW comes from lrmoe_compact_weighted. The results equal lrmoe_grouped_gemm_bwd's on
 * Dlt[c] = alpha[j] G[t] up to rounding: alpha scales the fp32 products instead of the
 * stored gradient rows, and in dW2 the rounding moves onto PhiW. A packed row whose t is
 * outside [0, T) contributes nothing (zero gradient row); j outside [0, N) reads zero
 * weight and zero [gate | up]. For swiglu = 0: dIn = dPhi [K_tot x F] and dH, X, H, W1, dW1
 * must be NULL. T * D * element size must be under 2 GiB (else LRMOE_ERR_UNSUPPORTED).
 * Workspace: as lrmoe_grouped_gemm_bwd in PHYSICAL mode. accumulate and din_ready as
 * there. */
lrmoe_status lrmoe_grouped_gemm_bwd_gathered(const lrmoe_problem* p, const int64_t* cseg_off_d, const void* G,
                                             const float* alpha, const int32_t* sel, const int32_t* ctok,
                                             const void* PhiW, const void* X, const void* H, const void* W2,
                                             const void* W1, float* dW2, float* dW1, void* dH, void* dIn,
                                             int32_t accumulate, void* ws, size_t ws_bytes, lrmoe_stream_t stream,
                                             lrmoe_event_t din_ready);

/* The forward that produces the backward's saved context (Algorithm 1's
 * FullForwardAndSaveContext; section 3.1: the forward keeps every routed pair). For every
 * pair j < N, expert-major (expert e: j in [seg_off[e], seg_off[e+1])), with t = tok[j]:
 *   H[j]   = X[t] W1[e]                    [gate | up], storage dtype [N x 2F], out
 *   Phi[j] = silu(gate) * up               from the fp32 sums, storage dtype [N x F], out
 *   Y[j]   = alpha[j] * (Phi[j] W2[e])     the stored Phi; storage dtype [N x D], out
 * bf16 MFMA with fp32 accumulation, one rounding per stored value. The layer output is
 * the token sum of the Y rows: lrmoe_scatter (TOKEN mode) with rows = Y, ctok = tok and
 * cslot = the pairs' slots. H and Phi are the saved activations lrmoe_score, lrmoe_compact
 * and lrmoe_grouped_gemm_bwd read. seg_off_d [E+1] int64 is the device copy of
 * p->seg_off. SwiGLU bf16 problems only (else LRMOE_ERR_UNSUPPORTED); X must be under
 * 2 GiB, as must each expert's W1 and W2 slice (32-bit offsets), else
 * LRMOE_ERR_UNSUPPORTED. p's quotas are checked but not used. No workspace. */
lrmoe_status lrmoe_expert_forward(const lrmoe_problem* p, const int64_t* seg_off_d, const void* X,
                                  const int32_t* tok, const float* alpha, const void* W1, const void* W2,
                                  void* H, void* Phi, void* Y, lrmoe_stream_t stream);

/* Step 5 - inverse mapping (section 3.1; Algorithm 1's ScatterWithZeros).
 * rows [n_rows x width] of dtype rows_dtype; row c belongs to pair (ctok[c], cslot[c]),
 * ctok in [0,T), cslot in [0,K), each (token, slot) at most once. Rows with an
 * out-of-range index are ignored.
 * TOKEN, TOKEN_BESIDE: out [T x width] f32 = per-token sums, added in slot order
 * (deterministic; the two modes give the same bits).
 * SLOT:  out [T*K x width] f32 = the row of each (t, k), zero where no row maps.
 * out is overwritten. pmap (may be NULL): the (token, slot) -> packed row map lrmoe_select
 * wrote for these rows (then n_rows must be K_tot, ctok and cslot may be NULL and no
 * workspace is needed); NULL: the map is built in ws from ctok and cslot. */
lrmoe_status lrmoe_scatter(const lrmoe_problem* p, lrmoe_scatter_mode mode, int64_t n_rows, int32_t width,
                           int32_t rows_dtype, const void* rows, const int32_t* ctok, const int32_t* cslot,
                           const int32_t* pmap, float* out, void* ws, size_t ws_bytes, lrmoe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LRMOE_H */
