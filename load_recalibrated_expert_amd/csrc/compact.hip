// Step 3: physical compaction (LRMoE paper, section 3.1 "compact runtime" and section 3.4,
// Figure 4). Retained gradient rows and their saved activations are gathered into
// contiguous expert segments so the grouped GEMMs see only retained rows, with no
// padding. Row c of every packed buffer belongs to the retained pair j = sel[c]. Two forms:
//   - weighted saved rows only: PhiW[c] = alpha_j * Phi[j] (the grouped GEMMs then read the
//     gradient rows g_{tok_j} by token and H[j] by pair; the routing weight sits on Phi,
//     which the FC2 weight gradient's bilinearity allows, appendix 7.1 Eq. 6-8);
//   - weighted gradient rows: Dlt[c] = alpha_j * g_{tok_j} (the weighted cotangent,
//     appendix 7.1 Eq. 5; alpha is applied here exactly once), and on request
//     PhiC[c] = Phi[j], XC[c] = X[tok_j], HC[c] = H[j] (the grouped GEMM can instead read
//     Phi, X and H in place through sel and ctok).
// The zero-masked baseline of section 3.4 keeps all N rows and zeroes the dropped pairs'
// gradient rows instead.
//
// HBM-bound gather/copy with 16-byte vector accesses, several loads in flight per lane
// before the matching stores. Physical compaction runs token-major through a [T x K] map
// from (token, slot) to packed row (each position holds at most one pair): the selection
// writes it, with ctok and cslot, when asked to; otherwise it is built here first. Then one
// wavefront per token writes all of its retained rows. Every pair of a token gathers
// the same G and X rows, so they come from HBM once and from L2 for the other pairs; in
// packed-row order the pairs of a token lie in different expert segments and each would
// fetch the rows again. The zero-masked baseline keeps pair order, one wavefront per row.
#include "common.h"

namespace lrmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;
constexpr int kU = 4;

__device__ __forceinline__ uint4 scale_bf16x8(float a, uint4 g) {
  uint4 o;
  o.x = mul_to_bf16(a, bf16_lo(g.x)) | (mul_to_bf16(a, bf16_hi(g.x)) << 16);
  o.y = mul_to_bf16(a, bf16_lo(g.y)) | (mul_to_bf16(a, bf16_hi(g.y)) << 16);
  o.z = mul_to_bf16(a, bf16_lo(g.z)) | (mul_to_bf16(a, bf16_hi(g.z)) << 16);
  o.w = mul_to_bf16(a, bf16_lo(g.w)) | (mul_to_bf16(a, bf16_hi(g.w)) << 16);
  return o;
}

__device__ __forceinline__ uint4 scale_f32x4(float a, uint4 g) {
  uint4 o;
  o.x = __float_as_uint(a * __uint_as_float(g.x));
  o.y = __float_as_uint(a * __uint_as_float(g.y));
  o.z = __float_as_uint(a * __uint_as_float(g.z));
  o.w = __float_as_uint(a * __uint_as_float(g.w));
  return o;
}

// dst[0..n) = src[0..n), 16-byte chunks strided over the wavefront. STREAM marks rows read
// once (Phi, H); token rows (X) stay cacheable for the token's other pairs.
template <bool STREAM>
__device__ __forceinline__ void copy_row(uint4* __restrict__ dst, const uint4* __restrict__ src, int n, int lane) {
  for (int c0 = lane; c0 < n; c0 += kWave * kU) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * kWave;
      if (c < n) v[u] = STREAM ? ld_stream(src + c) : src[c];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * kWave;
      if (c < n) dst[c] = v[u];
    }
  }
}

// Writes packed row c of pair j (token t): Dlt, and those of PhiC, XC (gated), HC (gated)
// that are given (never PhiC or HC when MASKED).
template <bool BF16, bool SWIGLU, bool MASKED>
__device__ __forceinline__ void gather_row(int64_t c, int64_t j, int t, bool tok_ok, bool kept, float a, int dch,
                                           int fch, int lane, const uint4* __restrict__ G,
                                           const uint4* __restrict__ Phi, const uint4* __restrict__ X,
                                           const uint4* __restrict__ H, uint4* __restrict__ Dlt,
                                           uint4* __restrict__ PhiC, uint4* __restrict__ XC,
                                           uint4* __restrict__ HC) {
  {  // weighted gradient row
    const uint4* src = G + (int64_t)t * dch;
    uint4* dst = Dlt + c * dch;
    for (int c0 = lane; c0 < dch; c0 += kWave * kU) {
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int cc = c0 + u * kWave;
        v[u] = (cc < dch && kept && tok_ok) ? src[cc] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int cc = c0 + u * kWave;
        if (cc < dch) dst[cc] = BF16 ? scale_bf16x8(a, v[u]) : scale_f32x4(a, v[u]);
      }
    }
  }
  if (!MASKED) {
    if (PhiC != nullptr) copy_row<true>(PhiC + c * fch, Phi + j * fch, fch, lane);
    if (SWIGLU && HC != nullptr) copy_row<true>(HC + c * 2 * fch, H + j * 2 * fch, 2 * fch, lane);
  }
  if (SWIGLU && XC != nullptr) {
    if (tok_ok) copy_row<false>(XC + c * dch, X + (int64_t)t * dch, dch, lane);
  }
}

// Zero-masked baseline: one wavefront per pair row, in pair order.
template <bool BF16, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void compact_masked_kernel(
    int64_t rows, int T, int dch, int fch, const uint8_t* __restrict__ keep, const uint4* __restrict__ G,
    const uint4* __restrict__ X, const float* __restrict__ alpha, const int32_t* __restrict__ tok,
    const int32_t* __restrict__ slot, uint4* __restrict__ Dlt, uint4* __restrict__ XC,
    int32_t* __restrict__ ctok, int32_t* __restrict__ cslot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t c = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (c >= rows) return;  // whole wavefront
  const int t = tok[c];
  const bool tok_ok = t >= 0 && t < T;
  gather_row<BF16, SWIGLU, true>(c, c, t, tok_ok, keep[c] != 0, alpha[c], dch, fch, lane, G, nullptr, X, nullptr,
                                 Dlt, nullptr, XC, nullptr);
  if (lane == 0) {
    if (ctok) ctok[c] = t;
    if (cslot) cslot[c] = slot[c];
  }
}

__global__ __launch_bounds__(kThreads) void position_fill_kernel(int64_t n, int32_t* __restrict__ map) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) map[i] = -1;
}

// For packed row c (pair j = sel[c]): ctok[c] = tok[j], cslot[c] = slot[j], and
// map[tok * K + slot] = c. A pair whose token or slot is out of range has no position:
// ctok[c] = cslot[c] = -1 and no map entry (its packed rows are zeroed by the compaction
// launch).
__global__ __launch_bounds__(kThreads) void position_map_kernel(int64_t rows, int64_t N, int T, int K,
                                                                const int32_t* __restrict__ sel,
                                                                const int32_t* __restrict__ tok,
                                                                const int32_t* __restrict__ slot,
                                                                int32_t* __restrict__ map, int32_t* __restrict__ ctok,
                                                                int32_t* __restrict__ cslot) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= rows) return;
  const int64_t j = sel[c];
  const bool pair_ok = j >= 0 && j < N;
  const int t = pair_ok ? tok[j] : -1, k = pair_ok ? slot[j] : -1;
  const bool valid = t >= 0 && t < T && k >= 0 && k < K;
  ctok[c] = valid ? t : -1;
  cslot[c] = valid ? k : -1;
  if (valid) map[(int64_t)t * K + k] = (int32_t)c;
}

// Zeroes the packed rows of retained pairs that have no (token, slot) position (ctok < 0):
// token-major compaction never reaches them. Block u of this part of a compaction grid
// scans packed rows [u * kFixRows, (u+1) * kFixRows), a wavefront 1024 of them; every
// flagged row is cleared by the whole wavefront.
constexpr int kFixRows = 4096;

__device__ __forceinline__ void zero_unmapped_rows(int u, int64_t rows, const int32_t* __restrict__ ctok, int dch,
                                                   int fch, bool swiglu, uint4* __restrict__ Dlt,
                                                   uint4* __restrict__ PhiC, uint4* __restrict__ XC,
                                                   uint4* __restrict__ HC) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t base = (int64_t)u * kFixRows + (int64_t)wave * (kFixRows / kRowsPerBlock);
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int i = 0; i < kFixRows / kRowsPerBlock / kWave; ++i) {
    const int64_t c = base + (int64_t)i * kWave + lane;
    uint64_t m = __ballot(c < rows && ctok[c] < 0);
    while (m) {  // uniform
      const int b = __builtin_ctzll(m);
      m &= m - 1;
      const int64_t r = base + (int64_t)i * kWave + b;
      for (int cc = lane; cc < dch; cc += kWave) {
        Dlt[r * dch + cc] = z;
        if (swiglu && XC != nullptr) XC[r * dch + cc] = z;
      }
      if (PhiC != nullptr)
        for (int cc = lane; cc < fch; cc += kWave) PhiC[r * fch + cc] = z;
      if (swiglu && HC != nullptr)
        for (int cc = lane; cc < 2 * fch; cc += kWave) HC[r * 2 * fch + cc] = z;
    }
  }
}

// Physical compaction, one wavefront per token: every retained row of the token in slot order.
// Generic shapes: each row is gathered section by section.
template <bool BF16, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void compact_token_kernel(
    int T, int K, int dch, int fch, int64_t rows, int tblocks, const int32_t* __restrict__ map,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ ctok, const uint4* __restrict__ G,
    const uint4* __restrict__ Phi, const uint4* __restrict__ X, const uint4* __restrict__ H,
    const float* __restrict__ alpha, uint4* __restrict__ Dlt, uint4* __restrict__ PhiC, uint4* __restrict__ XC,
    uint4* __restrict__ HC) {
  if ((int)blockIdx.x >= tblocks) {  // uniform per block
    zero_unmapped_rows((int)blockIdx.x - tblocks, rows, ctok, dch, fch, SWIGLU, Dlt, PhiC, XC, HC);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (t >= T) return;  // whole wavefront
  for (int k = 0; k < K; ++k) {
    const int32_t c = __builtin_amdgcn_readfirstlane(map[(int64_t)t * K + k]);
    if (c < 0) continue;
    const int64_t j = __builtin_amdgcn_readfirstlane(sel[c]);
    gather_row<BF16, SWIGLU, false>(c, j, t, true, true, alpha[j], dch, fch, lane, G, Phi, X, H, Dlt, PhiC, XC,
                                    HC);
  }
}

// Same rows for shapes whose rows fit the registers (dch <= 64 DL, fch <= 64 FL chunks): the
// token's G and X rows are loaded once and kept in registers, and the next pair's Phi and
// H rows are loaded before the current pair's rows are stored, so loads never queue behind
// the stores of the same pair (vector memory operations complete in issue order).
template <bool BF16, bool SWIGLU, int DL, int FL>
__global__ __launch_bounds__(kThreads) void compact_token_reg_kernel(
    int T, int K, int dch, int fch, int64_t rows, int tblocks, const int32_t* __restrict__ map,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ ctok, const uint4* __restrict__ G,
    const uint4* __restrict__ Phi, const uint4* __restrict__ X, const uint4* __restrict__ H,
    const float* __restrict__ alpha, uint4* __restrict__ Dlt, uint4* __restrict__ PhiC, uint4* __restrict__ XC,
    uint4* __restrict__ HC) {
  if ((int)blockIdx.x >= tblocks) {  // uniform per block
    zero_unmapped_rows((int)blockIdx.x - tblocks, rows, ctok, dch, fch, SWIGLU, Dlt, PhiC, XC, HC);
    return;
  }
  constexpr int HL = SWIGLU ? 2 * FL : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (t >= T) return;  // whole wavefront
  const int hch = 2 * fch;
  // next retained slot at or after k (K when none)
  auto next_slot = [&](int k) {
    for (; k < K; ++k)
      if (__builtin_amdgcn_readfirstlane(map[(int64_t)t * K + k]) >= 0) return k;
    return K;
  };
  int k = next_slot(0);
  if (k >= K) return;
  const bool with_phi = PhiC != nullptr, with_xc = SWIGLU && XC != nullptr, with_hc = SWIGLU && HC != nullptr;
  uint4 g[DL], x[SWIGLU ? DL : 1];
#pragma unroll
  for (int u = 0; u < DL; ++u) {
    const int cc = lane + u * kWave;
    g[u] = cc < dch ? G[(int64_t)t * dch + cc] : make_uint4(0, 0, 0, 0);
    if (with_xc) x[u] = cc < dch ? X[(int64_t)t * dch + cc] : make_uint4(0, 0, 0, 0);
  }
  int32_t c = __builtin_amdgcn_readfirstlane(map[(int64_t)t * K + k]);
  int64_t j = __builtin_amdgcn_readfirstlane(sel[c]);
  uint4 ph[FL], hh[HL];
  if (with_phi) {
#pragma unroll
    for (int u = 0; u < FL; ++u) {
      const int cc = lane + u * kWave;
      ph[u] = cc < fch ? ld_stream(Phi + j * fch + cc) : make_uint4(0, 0, 0, 0);
    }
  }
  if (with_hc) {
#pragma unroll
    for (int u = 0; u < HL; ++u) {
      const int cc = lane + u * kWave;
      hh[u] = cc < hch ? ld_stream(H + j * hch + cc) : make_uint4(0, 0, 0, 0);
    }
  }
  while (true) {
    const float a = alpha[j];
    const int kn = next_slot(k + 1);
    int32_t cn = -1;
    int64_t jn = 0;
    uint4 phn[FL], hhn[HL];
    if (kn < K) {  // uniform
      cn = __builtin_amdgcn_readfirstlane(map[(int64_t)t * K + kn]);
      jn = __builtin_amdgcn_readfirstlane(sel[cn]);
      if (with_phi) {
#pragma unroll
        for (int u = 0; u < FL; ++u) {
          const int cc = lane + u * kWave;
          phn[u] = cc < fch ? ld_stream(Phi + jn * fch + cc) : make_uint4(0, 0, 0, 0);
        }
      }
      if (with_hc) {
#pragma unroll
        for (int u = 0; u < HL; ++u) {
          const int cc = lane + u * kWave;
          hhn[u] = cc < hch ? ld_stream(H + jn * hch + cc) : make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < DL; ++u) {
      const int cc = lane + u * kWave;
      if (cc < dch) {
        Dlt[(int64_t)c * dch + cc] = BF16 ? scale_bf16x8(a, g[u]) : scale_f32x4(a, g[u]);
        if (with_xc) XC[(int64_t)c * dch + cc] = x[u];
      }
    }
    if (with_phi) {
#pragma unroll
      for (int u = 0; u < FL; ++u) {
        const int cc = lane + u * kWave;
        if (cc < fch) PhiC[(int64_t)c * fch + cc] = ph[u];
      }
    }
    if (with_hc) {
#pragma unroll
      for (int u = 0; u < HL; ++u) {
        const int cc = lane + u * kWave;
        if (cc < hch) HC[(int64_t)c * hch + cc] = hh[u];
      }
    }
    if (kn >= K) break;
    k = kn;
    c = cn;
    j = jn;
    if (with_phi) {
#pragma unroll
      for (int u = 0; u < FL; ++u) ph[u] = phn[u];
    }
    if (with_hc) {
#pragma unroll
      for (int u = 0; u < HL; ++u) hh[u] = hhn[u];
    }
  }
}

// Gradient rows only (the saved rows are read in place by the GEMMs), one wavefront per
// token, for K <= 64 slots and rows of at most DL x 64 16-byte chunks. All of the token's
// bookkeeping loads run lane-parallel (lane k: the packed row of slot k, its pair and
// alpha), three dependent round trips in all, while its G row loads into registers; then
// every retained slot's row is written from the registers.
template <bool BF16, int DL>
__global__ __launch_bounds__(kThreads) void compact_dlt_kernel(int T, int K, int dch, int64_t rows, int tblocks,
                                                               const int32_t* __restrict__ map,
                                                               const int32_t* __restrict__ sel,
                                                               const int32_t* __restrict__ ctok,
                                                               const uint4* __restrict__ G,
                                                               const float* __restrict__ alpha,
                                                               uint4* __restrict__ Dlt) {
  if ((int)blockIdx.x >= tblocks) {  // uniform per block
    zero_unmapped_rows((int)blockIdx.x - tblocks, rows, ctok, dch, 0, false, Dlt, nullptr, nullptr, nullptr);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (t >= T) return;  // whole wavefront
  uint4 g[DL];
#pragma unroll
  for (int u = 0; u < DL; ++u) {
    const int cc = lane + u * kWave;
    g[u] = cc < dch ? G[(int64_t)t * dch + cc] : make_uint4(0, 0, 0, 0);
  }
  const int32_t c = lane < K ? map[(int64_t)t * K + lane] : -1;
  const int64_t j = c >= 0 ? (int64_t)sel[c] : -1;
  const float a = j >= 0 ? alpha[j] : 0.0f;
  for (int k = 0; k < K; ++k) {
    const int32_t ck = __builtin_amdgcn_readlane(c, k);
    if (ck < 0) continue;  // uniform
    const float ak = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), k));
    uint4* dst = Dlt + (int64_t)ck * dch;
#pragma unroll
    for (int u = 0; u < DL; ++u) {
      const int cc = lane + u * kWave;
      if (cc < dch) dst[cc] = BF16 ? scale_bf16x8(ak, g[u]) : scale_f32x4(ak, g[u]);
    }
  }
}

// Weighted saved rows for the path that reads gradient rows by token: PhiW[c] =
// alpha_j * Phi[j] for j = sel[c] (one rounding to the storage dtype), a pair outside [0, N)
// giving a zero row. A block covers kWRows packed rows as one run of 16-byte chunks, so
// consecutive lanes read and write consecutive chunks of a row and rows follow each other
// without gaps; each thread keeps kU chunks in flight.
constexpr int kWRows = 16;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void compact_weighted_phi_kernel(int64_t rows, int64_t N, int fch,
                                                                        const int32_t* __restrict__ sel,
                                                                        const uint4* __restrict__ Phi,
                                                                        const float* __restrict__ alpha,
                                                                        uint4* __restrict__ PhiW) {
  const int64_t r0 = (int64_t)blockIdx.x * kWRows;
  const int nr = (int)min<int64_t>(kWRows, rows - r0);
  const int n = nr * fch;  // chunks of this block
  for (int l0 = threadIdx.x; l0 < n; l0 += kThreads * kU) {
    uint4 v[kU];
    float a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int l = l0 + u * kThreads;
      const int r = l / fch, ch = l - r * fch;
      const int64_t j = l < n ? (int64_t)sel[r0 + r] : -1;
      const bool ok = j >= 0 && j < N;
      a[u] = ok ? alpha[j] : 0.0f;
      v[u] = ok ? ld_stream(Phi + j * fch + ch) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int l = l0 + u * kThreads;
      if (l < n) PhiW[r0 * fch + l] = BF16 ? scale_bf16x8(a[u], v[u]) : scale_f32x4(a[u], v[u]);
    }
  }
}

template <bool BF16, bool SWIGLU>
void launch(int64_t rows, bool masked, const lrmoe_problem* p, const int32_t* sel, const uint8_t* keep,
            const void* G, const void* Phi, const void* X, const void* H, const float* alpha, const int32_t* tok,
            const int32_t* slot, void* Dlt, void* PhiC, void* XC, void* HC, int32_t* ctok, int32_t* cslot,
            const int32_t* pmap, int32_t* map, hipStream_t s) {
  const int esz = BF16 ? 2 : 4;
  const int dch = p->D * esz / 16, fch = p->F * esz / 16;
  if (masked) {
    compact_masked_kernel<BF16, SWIGLU><<<(unsigned)ceil_div(rows, kRowsPerBlock), kThreads, 0, s>>>(
        rows, p->T, dch, fch, keep, (const uint4*)G, (const uint4*)X, alpha, tok, slot, (uint4*)Dlt, (uint4*)XC, ctok,
        cslot);
    return;
  }
  if (pmap == nullptr) {  // build the (token, slot) map here, with ctok and cslot
    const int64_t positions = (int64_t)p->T * p->K;
    position_fill_kernel<<<(unsigned)ceil_div(positions, kThreads), kThreads, 0, s>>>(positions, map);
    position_map_kernel<<<(unsigned)ceil_div(rows, kThreads), kThreads, 0, s>>>(rows, p->N, p->T, p->K, sel, tok,
                                                                                slot, map, ctok, cslot);
    pmap = map;
  }
  const int tblocks = (int)ceil_div(p->T, kRowsPerBlock);
  const unsigned grid = (unsigned)(tblocks + ceil_div(rows, kFixRows));
  const bool dlt_only = PhiC == nullptr && XC == nullptr && HC == nullptr;
  if (dlt_only && p->K <= kWave && dch <= 4 * kWave)
    compact_dlt_kernel<BF16, 4><<<grid, kThreads, 0, s>>>(p->T, p->K, dch, rows, tblocks, pmap, sel, ctok,
                                                           (const uint4*)G, alpha, (uint4*)Dlt);
  else if (dlt_only && p->K <= kWave && dch <= 8 * kWave)
    compact_dlt_kernel<BF16, 8><<<grid, kThreads, 0, s>>>(p->T, p->K, dch, rows, tblocks, pmap, sel, ctok,
                                                           (const uint4*)G, alpha, (uint4*)Dlt);
  else if (dch <= 4 * kWave && fch <= 2 * kWave)
    compact_token_reg_kernel<BF16, SWIGLU, 4, 2><<<grid, kThreads, 0, s>>>(
        p->T, p->K, dch, fch, rows, tblocks, pmap, sel, ctok, (const uint4*)G, (const uint4*)Phi, (const uint4*)X,
        (const uint4*)H, alpha, (uint4*)Dlt, (uint4*)PhiC, (uint4*)XC, (uint4*)HC);
  else
    compact_token_kernel<BF16, SWIGLU><<<grid, kThreads, 0, s>>>(
        p->T, p->K, dch, fch, rows, tblocks, pmap, sel, ctok, (const uint4*)G, (const uint4*)Phi, (const uint4*)X,
        (const uint4*)H, alpha, (uint4*)Dlt, (uint4*)PhiC, (uint4*)XC, (uint4*)HC);
}

}  // namespace

lrmoe_status launch_compact_weighted_phi(const lrmoe_problem* p, int64_t rows, const int32_t* sel,
                                         const void* Phi, const float* alpha, void* PhiW, hipStream_t s) {
  if (rows <= 0) return LRMOE_OK;
  const bool bf16 = p->dtype == LRMOE_BF16;
  const int fch = p->F * (bf16 ? 2 : 4) / 16;
  const unsigned grid = (unsigned)ceil_div(rows, kWRows);
  if (bf16)
    compact_weighted_phi_kernel<true><<<grid, kThreads, 0, s>>>(rows, p->N, fch, sel, (const uint4*)Phi, alpha,
                                                                (uint4*)PhiW);
  else
    compact_weighted_phi_kernel<false><<<grid, kThreads, 0, s>>>(rows, p->N, fch, sel, (const uint4*)Phi, alpha,
                                                                 (uint4*)PhiW);
  return launch_status();
}

size_t compact_ws_bytes(const lrmoe_problem* p) { return align_up(sizeof(int32_t) * (size_t)p->T * p->K, 256); }

lrmoe_status launch_compact(const lrmoe_problem* p, int64_t rows, bool masked, const int32_t* sel,
                            const uint8_t* keep, const void* G, const void* Phi, const void* X,
                            const void* H, const float* alpha, const int32_t* tok, const int32_t* slot,
                            void* Dlt, void* PhiC, void* XC, void* HC, int32_t* ctok, int32_t* cslot,
                            const int32_t* pmap, void* ws, hipStream_t s) {
  if (rows <= 0) return LRMOE_OK;
  const bool bf16 = p->dtype == LRMOE_BF16, sw = p->swiglu != 0;
  int32_t* map = (int32_t*)ws;
#define LRMOE_COMPACT_CASE(B, S)                                                                               \
  if (bf16 == B && sw == S)                                                                                    \
    launch<B, S>(rows, masked, p, sel, keep, G, Phi, X, H, alpha, tok, slot, Dlt, PhiC, XC, HC, ctok, cslot, pmap, \
                 map, s);
  LRMOE_COMPACT_CASE(true, true)
  LRMOE_COMPACT_CASE(true, false)
  LRMOE_COMPACT_CASE(false, true)
  LRMOE_COMPACT_CASE(false, false)
#undef LRMOE_COMPACT_CASE
  return launch_status();
}

}  // namespace lrmoe
