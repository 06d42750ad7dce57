// Step 3: physical compaction (LRMoE paper, section 3.1 "compact runtime" and section 3.4,
// Figure 4). Retained gradient rows and their saved activations are gathered into
// contiguous expert segments so the grouped GEMMs see only retained rows, with no
// padding. Row c of every packed buffer belongs to the retained pair j = sel[c]:
//   Dlt[c] = alpha_j * g_{tok_j} (the weighted cotangent, appendix 7.1 Eq. 5; alpha is
//   applied here exactly once), PhiC[c] = Phi[j], XC[c] = X[tok_j], HC[c] = H[j].
// The zero-masked baseline of section 3.4 keeps all N rows and zeroes the dropped pairs'
// gradient rows instead.
//
// HBM-bound gather/copy: one wavefront per packed row, 16-byte vector accesses, several
// loads in flight per lane before the matching stores.
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

// dst[0..n) = src[0..n), 16-byte chunks strided over the wavefront.
__device__ __forceinline__ void copy_row(uint4* __restrict__ dst, const uint4* __restrict__ src, int n, int lane) {
  for (int c0 = lane; c0 < n; c0 += kWave * kU) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * kWave;
      if (c < n) v[u] = ld_stream(src + c);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * kWave;
      if (c < n) dst[c] = v[u];
    }
  }
}

template <bool BF16, bool SWIGLU, bool MASKED>
__global__ __launch_bounds__(kThreads) void compact_kernel(
    int64_t rows, int64_t N, int T, int dch, int fch, const int32_t* __restrict__ sel, const uint8_t* __restrict__ keep,
    const uint4* __restrict__ G, const uint4* __restrict__ Phi, const uint4* __restrict__ X,
    const uint4* __restrict__ H, const float* __restrict__ alpha, const int32_t* __restrict__ tok,
    const int32_t* __restrict__ slot, uint4* __restrict__ Dlt, uint4* __restrict__ PhiC, uint4* __restrict__ XC,
    uint4* __restrict__ HC, int32_t* __restrict__ ctok, int32_t* __restrict__ cslot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t c = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (c >= rows) return;  // whole wavefront
  const int64_t j = MASKED ? c : (int64_t)sel[c];
  if (j < 0 || j >= N) return;  // not a pair index: nothing to gather
  const int t = tok[j];
  const bool tok_ok = t >= 0 && t < T;
  const bool kept = MASKED ? (keep[j] != 0) : true;
  const float a = alpha[j];
  // weighted gradient row
  {
    const uint4* src = G + (int64_t)t * dch;
    uint4* dst = Dlt + c * dch;
    for (int c0 = lane; c0 < dch; c0 += kWave * kU) {
      uint4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int cc = c0 + u * kWave;
        v[u] = (cc < dch && kept && tok_ok) ? ld_stream(src + cc) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int cc = c0 + u * kWave;
        if (cc < dch) dst[cc] = BF16 ? scale_bf16x8(a, v[u]) : scale_f32x4(a, v[u]);
      }
    }
  }
  if (!MASKED) {
    copy_row(PhiC + c * fch, Phi + j * fch, fch, lane);
    if (SWIGLU) copy_row(HC + c * 2 * fch, H + j * 2 * fch, 2 * fch, lane);
  }
  if (SWIGLU) {
    if (tok_ok) copy_row(XC + c * dch, X + (int64_t)t * dch, dch, lane);
  }
  if (lane == 0) {
    if (ctok) ctok[c] = t;
    if (cslot) cslot[c] = slot[j];
  }
}

template <bool BF16, bool SWIGLU, bool MASKED>
void launch(int64_t rows, const lrmoe_problem* p, const int32_t* sel, const uint8_t* keep, const void* G,
            const void* Phi, const void* X, const void* H, const float* alpha, const int32_t* tok,
            const int32_t* slot, void* Dlt, void* PhiC, void* XC, void* HC, int32_t* ctok, int32_t* cslot,
            hipStream_t s) {
  const int esz = BF16 ? 2 : 4;
  const int dch = p->D * esz / 16, fch = p->F * esz / 16;
  compact_kernel<BF16, SWIGLU, MASKED><<<(unsigned)ceil_div(rows, kRowsPerBlock), kThreads, 0, s>>>(
      rows, p->N, p->T, dch, fch, sel, keep, (const uint4*)G, (const uint4*)Phi, (const uint4*)X, (const uint4*)H,
      alpha, tok, slot, (uint4*)Dlt, (uint4*)PhiC, (uint4*)XC, (uint4*)HC, ctok, cslot);
}

}  // namespace

lrmoe_status launch_compact(const lrmoe_problem* p, int64_t rows, bool masked, const int32_t* sel,
                            const uint8_t* keep, const void* G, const void* Phi, const void* X,
                            const void* H, const float* alpha, const int32_t* tok, const int32_t* slot,
                            void* Dlt, void* PhiC, void* XC, void* HC, int32_t* ctok, int32_t* cslot,
                            hipStream_t s) {
  if (rows <= 0) return LRMOE_OK;
  const bool bf16 = p->dtype == LRMOE_BF16, sw = p->swiglu != 0;
#define LRMOE_COMPACT_CASE(B, S, M)                                                                      \
  if (bf16 == B && sw == S && masked == M)                                                               \
    launch<B, S, M>(rows, p, sel, keep, G, Phi, X, H, alpha, tok, slot, Dlt, PhiC, XC, HC, ctok, cslot, s);
  LRMOE_COMPACT_CASE(true, true, false)
  LRMOE_COMPACT_CASE(true, true, true)
  LRMOE_COMPACT_CASE(true, false, false)
  LRMOE_COMPACT_CASE(true, false, true)
  LRMOE_COMPACT_CASE(false, true, false)
  LRMOE_COMPACT_CASE(false, true, true)
  LRMOE_COMPACT_CASE(false, false, false)
  LRMOE_COMPACT_CASE(false, false, true)
#undef LRMOE_COMPACT_CASE
  return launch_status();
}

}  // namespace lrmoe
