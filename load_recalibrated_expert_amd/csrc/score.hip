// Step 1: LRM score of every routed pair (LRMoE paper, section 3.2, Proposition 3.1,
// Eq. 3): R_u = alpha_u^2 * ||g_t||^2 * ||phi_u||^2. Because the pair's weight-gradient
// contribution (alpha_u g_t) phi_u^T is rank one, its squared Frobenius norm factorises
// into two row norms, so the kernel never forms the outer product.
//
// HBM-bound streaming: token norms read G once ([T x D]); pair norms read Phi once
// ([N x F]) plus alpha/tok, gather ||g_t||^2 from an L2-resident [T] fp64 table and
// write R. Squares of bf16 values are exact in f32; sums run in fp64.
#include "common.h"

namespace lrmoe {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kUnroll = 4;

// One wavefront per token row; each lane streams 16-byte chunks. ABS: sum of magnitudes
// instead of squares (the absolute-gradient criterion of the ablation).
template <bool BF16, bool ABS = false>
__global__ __launch_bounds__(kScoreThreads) void token_sqnorm_kernel(const uint4* __restrict__ G,
                                                                     int T, int chunks_per_row,
                                                                     double* __restrict__ gn) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * (kScoreThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // the whole wavefront leaves together; no block-level sync follows
  const uint4* row = G + t * chunks_per_row;
  double acc = 0.0;
  for (int c0 = lane; c0 < chunks_per_row; c0 += kWave * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int c = c0 + u * kWave;
      v[u] = c < chunks_per_row ? ld_stream(row + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (ABS) acc += BF16 ? sumabs_bf16x8(v[u]) : sumabs_f32x4(v[u]);
      else acc += BF16 ? sumsq_bf16x8(v[u]) : sumsq_f32x4(v[u]);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) gn[t] = acc;
}

// Sixteen lanes per pair row (rows of the FC2 input are short); four rows per wavefront.
template <bool BF16>
__global__ __launch_bounds__(kScoreThreads) void pair_score_kernel(const uint4* __restrict__ Phi,
                                                                   const float* __restrict__ alpha,
                                                                   const int32_t* __restrict__ tok,
                                                                   const double* __restrict__ gn,
                                                                   int64_t N, int T, int chunks_per_row,
                                                                   float* __restrict__ R) {
  constexpr int kLanes = 16;
  const int sub = threadIdx.x & (kLanes - 1);
  const int64_t j = (int64_t)blockIdx.x * (kScoreThreads / kLanes) + threadIdx.x / kLanes;
  double acc = 0.0;
  if (j < N) {
    const uint4* row = Phi + j * chunks_per_row;
    for (int c0 = sub; c0 < chunks_per_row; c0 += kLanes * kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int c = c0 + u * kLanes;
        v[u] = c < chunks_per_row ? ld_stream(row + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc += BF16 ? sumsq_bf16x8(v[u]) : sumsq_f32x4(v[u]);
    }
  }
#pragma unroll
  for (int o = kLanes / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kLanes);
  if (sub == 0 && j < N) {
    const int t = tok[j];
    const double g = (t >= 0 && t < T) ? gn[t] : 0.0;  // out-of-range tokens score 0
    const double a = (double)alpha[j];
    R[j] = (float)(a * a * g * acc);
  }
}

// Gradient-only criteria (section 4.7, Table 2): every pair takes its token's row score.
__global__ __launch_bounds__(kScoreThreads) void pair_gather_kernel(const int32_t* __restrict__ tok,
                                                                    const double* __restrict__ gs, int64_t N,
                                                                    int T, float* __restrict__ R) {
  const int64_t j = (int64_t)blockIdx.x * kScoreThreads + threadIdx.x;
  if (j >= N) return;
  const int t = tok[j];
  R[j] = (t >= 0 && t < T) ? (float)gs[t] : 0.0f;  // out-of-range tokens score 0
}

}  // namespace

lrmoe_status launch_score_gradient(const lrmoe_problem* p, bool magnitude, const void* G, const int32_t* tok,
                                   float* R, double* gs, hipStream_t s) {
  const bool bf16 = p->dtype == LRMOE_BF16;
  const int gch = p->D * (bf16 ? 2 : 4) / 16;
  if (p->T > 0) {
    dim3 grid((unsigned)ceil_div(p->T, kScoreThreads / kWave));
    if (bf16 && magnitude) token_sqnorm_kernel<true, true><<<grid, kScoreThreads, 0, s>>>((const uint4*)G, p->T, gch, gs);
    else if (bf16) token_sqnorm_kernel<true, false><<<grid, kScoreThreads, 0, s>>>((const uint4*)G, p->T, gch, gs);
    else if (magnitude) token_sqnorm_kernel<false, true><<<grid, kScoreThreads, 0, s>>>((const uint4*)G, p->T, gch, gs);
    else token_sqnorm_kernel<false, false><<<grid, kScoreThreads, 0, s>>>((const uint4*)G, p->T, gch, gs);
  }
  if (p->N > 0)
    pair_gather_kernel<<<(unsigned)ceil_div(p->N, kScoreThreads), kScoreThreads, 0, s>>>(tok, gs, p->N, p->T, R);
  return launch_status();
}

lrmoe_status launch_score(const lrmoe_problem* p, const void* G, const void* Phi, const float* alpha,
                          const int32_t* tok, float* R, double* gn, hipStream_t s) {
  const bool bf16 = p->dtype == LRMOE_BF16;
  const int esz = bf16 ? 2 : 4;
  const int gch = p->D * esz / 16, pch = p->F * esz / 16;
  if (p->T > 0) {
    dim3 grid((unsigned)ceil_div(p->T, kScoreThreads / kWave));
    if (bf16)
      token_sqnorm_kernel<true><<<grid, kScoreThreads, 0, s>>>((const uint4*)G, p->T, gch, gn);
    else
      token_sqnorm_kernel<false><<<grid, kScoreThreads, 0, s>>>((const uint4*)G, p->T, gch, gn);
  }
  if (p->N > 0) {
    dim3 grid((unsigned)ceil_div(p->N, kScoreThreads / 16));
    if (bf16)
      pair_score_kernel<true><<<grid, kScoreThreads, 0, s>>>((const uint4*)Phi, alpha, tok, gn, p->N,
                                                             p->T, pch, R);
    else
      pair_score_kernel<false><<<grid, kScoreThreads, 0, s>>>((const uint4*)Phi, alpha, tok, gn, p->N,
                                                              p->T, pch, R);
  }
  return launch_status();
}

}  // namespace lrmoe
