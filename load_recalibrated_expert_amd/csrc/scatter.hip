// Step 5: inverse mapping (LRMoE paper, section 3.1 and Algorithm 1's ScatterWithZeros).
// Every packed input-gradient row goes back to the (token, slot) position its pair came
// from; positions whose pair was dropped stay zero, and the token-order output adds up the
// rows of each token.
//
// Each packed row belongs to one (token, slot) position and each position holds at most one
// pair, so a [T x K] map from position to packed row drives the scatter: the one the
// selection wrote, or one built here first (fill -1, then one store per row: no
// conflicts). Token mode then sums, per token, the rows of its K slots in slot order - a
// fixed order, so the result is deterministic without atomics. Slot mode copies each
// position's row or writes zeros.
#include <algorithm>
#include <atomic>

#include "common.h"

namespace lrmoe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void map_fill_kernel(int64_t n, int32_t* __restrict__ map) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) map[i] = -1;
}

__global__ __launch_bounds__(kThreads) void map_scatter_kernel(int64_t rows, int T, int K,
                                                               const int32_t* __restrict__ ctok,
                                                               const int32_t* __restrict__ cslot,
                                                               int32_t* __restrict__ map) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= rows) return;
  const int t = ctok[c], k = cslot[c];
  if (t >= 0 && t < T && k >= 0 && k < K) map[(int64_t)t * K + k] = (int32_t)c;
}

// 8 elements of a row -> f32, from 16 bytes (bf16) or 32 bytes (f32).
template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ rows, int64_t row, int width, int c8, float v[8]) {
  if (BF16) {
    const uint4 x = ld_stream((const uint4*)((const uint16_t*)rows + row * width) + c8);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const float4* p = (const float4*)((const float*)rows + row * width) + 2 * c8;
    const uint4 a = ld_stream(p), b = ld_stream(p + 1);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

__device__ __forceinline__ void store8(float* __restrict__ out, int64_t row, int width, int c8, const float v[8]) {
  float4* p = (float4*)(out + row * width) + 2 * c8;
  p[0] = make_float4(v[0], v[1], v[2], v[3]);
  p[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// out[t] = sum over k of rows[map[t][k]], in slot order, by one wavefront. The token's K map
// entries are read once (wave-uniform), and for K <= kMaxK the row chunks of CB column
// blocks are all loaded before the first add, so a lane keeps up to CB * K loads in
// flight; the adds still run in slot order, so CB does not change the result.
constexpr int kMaxK = 8;

template <bool BF16, int CB>
__device__ __forceinline__ void reduce_token(int64_t t, int K, int width, const int32_t* __restrict__ map,
                                             const void* __restrict__ rows, float* __restrict__ out, int lane) {
  const int n8 = width / 8;
  if (K <= kMaxK) {
    int32_t m[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) m[k] = k < K ? __builtin_amdgcn_readfirstlane(map[t * K + k]) : -1;
    constexpr int W = BF16 ? 1 : 2;  // 16-byte words per 8 elements
    for (int c0 = lane; c0 < n8; c0 += CB * kWave) {
      uint4 raw[CB][kMaxK][W];
#pragma unroll
      for (int u = 0; u < CB; ++u)
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
          const int c8 = c0 + u * kWave;
          const bool ok = m[k] >= 0 && c8 < n8;
#pragma unroll
          for (int q = 0; q < W; ++q)
            raw[u][k][q] = ok ? ld_stream((const uint4*)rows + ((int64_t)m[k] * width / 8 + c8) * W + q)
                              : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int c8 = c0 + u * kWave;
        if (c8 >= n8) break;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
          float v[8];
          if (BF16) {
            const uint32_t w[4] = {raw[u][k][0].x, raw[u][k][0].y, raw[u][k][0].z, raw[u][k][0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[2 * i] = bf16_lo(w[i]);
              v[2 * i + 1] = bf16_hi(w[i]);
            }
          } else {
            const uint32_t w[8] = {raw[u][k][0].x, raw[u][k][0].y, raw[u][k][0].z, raw[u][k][0].w,
                                   raw[u][k][W - 1].x, raw[u][k][W - 1].y, raw[u][k][W - 1].z, raw[u][k][W - 1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
        store8(out, t, width, c8, acc);
      }
    }
    return;
  }
  for (int c8 = lane; c8 < n8; c8 += kWave) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < K; ++k) {
      const int32_t r = map[t * K + k];
      if (r < 0) continue;
      float v[8];
      load8<BF16>(rows, r, width, c8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8(out, t, width, c8, acc);
  }
}

// One wavefront per token, two column blocks per pass (a standalone launch: every compute
// unit takes as many token waves as fit).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void token_reduce_kernel(int T, int K, int width,
                                                                const int32_t* __restrict__ map,
                                                                const void* __restrict__ rows,
                                                                float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (t >= T) return;
  reduce_token<BF16, 2>(t, K, width, map, rows, out, (int)threadIdx.x & (kWave - 1));
}

// The same sums from a grid of at most one block per compute unit, each wavefront looping
// over tokens with one column block per pass (bf16 rows: under 64 registers), for a scatter
// that runs on a second stream beside the weight-gradient launch: the gathered
// weight-gradient kernel's two wavefronts per SIMD leave 80 of the SIMD's 512 registers per
// lane, room for one such wavefront, so the scatter runs on the compute units the GEMM
// occupies instead of taking them over as they free up.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void token_reduce_beside_kernel(int T, int K, int width,
                                                                       const int32_t* __restrict__ map,
                                                                       const void* __restrict__ rows,
                                                                       float* __restrict__ out) {
  const int64_t step = (int64_t)gridDim.x * (kThreads / kWave);
  for (int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
       t < T; t += step)
    reduce_token<BF16, 1>(t, K, width, map, rows, out, (int)threadIdx.x & (kWave - 1));
}

// One wavefront per (token, slot) position: copy its row or write zeros.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void slot_copy_kernel(int64_t positions, int width,
                                                             const int32_t* __restrict__ map,
                                                             const void* __restrict__ rows,
                                                             float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t q = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (q >= positions) return;
  const int32_t r = map[q];
  const int n8 = width / 8;
  for (int c8 = lane; c8 < n8; c8 += kWave) {
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r >= 0) load8<BF16>(rows, r, width, c8, v);
    store8(out, q, width, c8, v);
  }
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // zero until looked up

// Compute units of the current device (looked up on the first call on that device).
lrmoe_status device_cu_count(int* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LRMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LRMOE_ERR_UNSUPPORTED;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return LRMOE_ERR_HIP;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return LRMOE_OK;
}

}  // namespace

size_t scatter_ws_bytes(const lrmoe_problem* p) { return align_up(sizeof(int32_t) * (size_t)p->T * p->K, 256); }

lrmoe_status launch_scatter(const lrmoe_problem* p, int mode, int64_t n_rows, int width, int rows_dtype,
                            const void* rows, const int32_t* ctok, const int32_t* cslot, const int32_t* pmap,
                            float* out, void* ws, hipStream_t s) {
  const int64_t positions = (int64_t)p->T * p->K;
  if (positions == 0) return LRMOE_OK;
  const int32_t* map = pmap;
  if (map == nullptr) {  // build the (token, slot) map from the rows' tokens and slots
    int32_t* m = (int32_t*)ws;
    map_fill_kernel<<<(unsigned)ceil_div(positions, kThreads), kThreads, 0, s>>>(positions, m);
    if (n_rows > 0)
      map_scatter_kernel<<<(unsigned)ceil_div(n_rows, kThreads), kThreads, 0, s>>>(n_rows, p->T, p->K, ctok,
                                                                                   cslot, m);
    map = m;
  }
  const bool bf16 = rows_dtype == LRMOE_BF16;
  constexpr int per_block = kThreads / kWave;
  if (mode == LRMOE_SCATTER_TOKEN) {
    const unsigned g = (unsigned)ceil_div(p->T, per_block);
    if (bf16) token_reduce_kernel<true><<<g, kThreads, 0, s>>>(p->T, p->K, width, map, rows, out);
    else token_reduce_kernel<false><<<g, kThreads, 0, s>>>(p->T, p->K, width, map, rows, out);
  } else if (mode == LRMOE_SCATTER_TOKEN_BESIDE) {
    int cus = 0;
    if (device_cu_count(&cus) != LRMOE_OK) return LRMOE_ERR_HIP;
    const unsigned g = (unsigned)std::min<int64_t>(ceil_div(p->T, per_block), cus);
    if (bf16) token_reduce_beside_kernel<true><<<g, kThreads, 0, s>>>(p->T, p->K, width, map, rows, out);
    else token_reduce_beside_kernel<false><<<g, kThreads, 0, s>>>(p->T, p->K, width, map, rows, out);
  } else {
    const unsigned g = (unsigned)ceil_div(positions, per_block);
    if (bf16) slot_copy_kernel<true><<<g, kThreads, 0, s>>>(positions, width, map, rows, out);
    else slot_copy_kernel<false><<<g, kThreads, 0, s>>>(positions, width, map, rows, out);
  }
  return launch_status();
}

}  // namespace lrmoe
