// Step 4: packed expert backward as variable-size grouped GEMMs (LRMoE paper, section 3.4:
// the FC2 and FC1 data- and weight-gradient GEMMs run on the retained rows only; the
// retained row count m_e of expert e is the row dimension of the data-gradient products
// and the reduction dimension of the weight-gradient products; section 3.1: the activation
// backward between FC2 and FC1 uses the same retained identities).
//
// Weights are stored [in x out]: W2[e] is [F x D], W1[e] is [D x 2F] ([gate | up]).
//   FC2 dgrad  dPhi = Dlt W2^T      both operands contiguous along the reduction (d)
//   SwiGLU     dH   = [dPhi*up*silu'(gate), dPhi*silu(gate)]   fused in the FC2 dgrad epilogue
//   FC1 dgrad  dIn  = dH W1^T       both operands contiguous along the reduction (j)
//   FC2 wgrad  dW2  = PhiC^T Dlt    reduction over the packed rows: operands are row-major
//   FC1 wgrad  dW1  = XC^T dH       in the output dims, transposed on the way into LDS
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulation. A block of 256 threads
// (four 64-wide wavefronts, 2x2) owns a 256x256 output tile; each wavefront a 128x128
// sub-tile held as 4x4 MFMA accumulators. K advances 64 per stage through two LDS stages
// (2 x 64 KB): the next stage's global loads are issued before the current stage's MFMAs
// and written to the other LDS stage after them, one barrier per stage. LDS rows are
// 128 bytes (64 bf16 along K) with the 16-byte chunk index XOR-swizzled by the row so
// 16-byte fragment reads spread over the banks. Weight-gradient tiles split the packed rows
// of large experts into K chunks; chunk partials go to the workspace and a second kernel
// sums them in chunk order, so results do not depend on scheduling. Blocks are renumbered
// so each XCD (hardware round-robins blocks over its 8 XCDs) walks a contiguous run of
// tiles that share operands in its L2.
//
// f32 path (small problems): plain fp32 FMA kernels, no bf16 anywhere.
#include "common.h"

namespace lrmoe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int kTileChunks = BM * BK / 8;  // uint4 per operand tile per stage
constexpr int64_t kKcMax = 16384;        // max packed rows per weight-gradient chunk

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, i = b >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + i;
}

// ---------------------------------------------------------------- global -> LDS staging

// Operand stored [rows x K] with K contiguous: tile rows [0, rows_valid), k in [k0, k0+64).
__device__ __forceinline__ void load_kc(const uint16_t* __restrict__ base, int64_t ld, int rows_valid, int k0,
                                        int kend, uint4 (&v)[8]) {
  const int ch = threadIdx.x & 7, r0 = threadIdx.x >> 3;
  const int k = k0 + ch * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 32 * i;
    v[i] = (r < rows_valid && k < kend) ? *(const uint4*)(base + (int64_t)r * ld + k) : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void store_kc(uint4* __restrict__ lds, const uint4 (&v)[8]) {
  const int ch = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 32 * i;
    lds[r * 8 + (ch ^ swz(r))] = v[i];
  }
}

// Operand stored [K x cols] with cols contiguous (row index = reduction index): tile
// columns [0, 256) of which [0, mn_valid) exist, reduction rows [k0, k0+64) below kend.
__device__ __forceinline__ void load_mn(const uint16_t* __restrict__ base, int64_t ld, int mn_valid, int k0,
                                        int kend, uint4 (&v)[8]) {
  const int mc = threadIdx.x & 31, kg = threadIdx.x >> 5;
  const bool col_ok = mc * 8 < mn_valid;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + kg * 8 + i;
    v[i] = (col_ok && k < kend) ? *(const uint4*)(base + (int64_t)k * ld + mc * 8) : make_uint4(0, 0, 0, 0);
  }
}
// 8x8 transpose of 16-bit values: v[k] holds columns m0..m7 of reduction row k; out row m
// holds reduction rows k0..k7 of column m, which is what an MFMA fragment wants.
__device__ __forceinline__ void store_mn(uint4* __restrict__ lds, const uint4 (&v)[8]) {
  const int mc = threadIdx.x & 31, kg = threadIdx.x >> 5;
  uint32_t w[8][4];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w[k][0] = v[k].x;
    w[k][1] = v[k].y;
    w[k][2] = v[k].z;
    w[k][3] = v[k].w;
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int p = m >> 1;
    const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
    uint4 o;
    o.x = __builtin_amdgcn_perm(w[1][p], w[0][p], sel);
    o.y = __builtin_amdgcn_perm(w[3][p], w[2][p], sel);
    o.z = __builtin_amdgcn_perm(w[5][p], w[4][p], sel);
    o.w = __builtin_amdgcn_perm(w[7][p], w[6][p], sel);
    const int r = mc * 8 + m;
    lds[r * 8 + (kg ^ swz(r))] = o;
  }
}

// ---------------------------------------------------------------- MFMA on one LDS stage

__device__ __forceinline__ void mma_stage(const uint4* __restrict__ la, const uint4* __restrict__ lb,
                                          f32x16_t (&acc)[4][4], int wm, int wn, int lane) {
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ch = kk * 2 + lk;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + lr;
      const int rb = wn * 128 + i * 32 + lr;
      a[i] = __builtin_bit_cast(bf16x8_t, la[ra * 8 + (ch ^ swz(ra))]);
      b[i] = __builtin_bit_cast(bf16x8_t, lb[rb * 8 + (ch ^ swz(rb))]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// acc[i][j][v] sits at tile row wm*128 + i*32 + 8*(v/4) + 4*(lane/32) + v%4,
// tile column wn*128 + j*32 + lane%32.
#define LRMOE_FOR_ACC(BODY)                                                               \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) _Pragma("unroll") for (int j = 0; j < 4; ++j) \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) {                                    \
    const int tr = wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);          \
    const int tc = wn * 128 + j * 32 + (lane & 31);                                       \
    const float val = acc[i][j][v];                                                       \
    BODY                                                                                  \
  }

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
}

// ---------------------------------------------------------------- data-gradient kernel

enum { EPI_SWIGLU = 0, EPI_STORE = 1 };

struct DgradArgs {
  const uint16_t* A;   // [rows x K] packed rows (Dlt or dH)
  int64_t lda;
  const uint16_t* W;   // [E x N x K] weights viewed as rows n with K contiguous
  int64_t ldw, w_estride;
  int N, K;            // output columns, reduction length
  int ntn;             // ceil(N / BN)
  const int64_t* row_off;
  int E;
  // epilogue
  const uint16_t* HC;  // SwiGLU: [rows x 2F] saved [gate | up]
  uint16_t* out;       // SwiGLU: dH [rows x 2F]; STORE: [rows x N]
  int64_t ldo;
  int F;
};

template <int EPI>
__global__ __launch_bounds__(NTHR) void dgrad_kernel(DgradArgs g) {
  __shared__ uint4 lds[2][2][kTileChunks];
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  // locate the tile: experts in order, ceil(m_e/BM) x ntn tiles each
  int e = 0, local = b;
  int64_t r0 = 0, m = 0;
  for (; e < g.E; ++e) {
    r0 = g.row_off[e];
    m = g.row_off[e + 1] - r0;
    const int cnt = (int)((m + BM - 1) / BM) * g.ntn;
    if (local < cnt) break;
    local -= cnt;
  }
  if (e >= g.E) return;  // cannot happen with a host-sized grid; uniform per block
  const int mt = local / g.ntn, nt = local % g.ntn;
  const int64_t row0 = r0 + (int64_t)mt * BM;
  const int rows_valid = (int)min<int64_t>(BM, m - (int64_t)mt * BM);
  const int n0 = nt * BN;
  const int n_valid = min(BN, g.N - n0);
  const uint16_t* Ab = g.A + row0 * g.lda;
  const uint16_t* Bb = g.W + (int64_t)e * g.w_estride + (int64_t)n0 * g.ldw;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[4][4];
  zero_acc(acc);
  uint4 ra[8], rb[8];
  const int nk = (g.K + BK - 1) / BK;
  load_kc(Ab, g.lda, rows_valid, 0, g.K, ra);
  load_kc(Bb, g.ldw, n_valid, 0, g.K, rb);
  store_kc(lds[0][0], ra);
  store_kc(lds[0][1], rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_kc(Ab, g.lda, rows_valid, (kt + 1) * BK, g.K, ra);
      load_kc(Bb, g.ldw, n_valid, (kt + 1) * BK, g.K, rb);
    }
    mma_stage(lds[cur][0], lds[cur][1], acc, wm, wn, lane);
    if (more) {
      store_kc(lds[cur ^ 1][0], ra);
      store_kc(lds[cur ^ 1][1], rb);
    }
    __syncthreads();
  }

  if (EPI == EPI_SWIGLU) {
    const int64_t ld = 2 * (int64_t)g.F;
    LRMOE_FOR_ACC({
      if (tr < rows_valid && tc < n_valid) {
        const int64_t row = row0 + tr;
        const int f = n0 + tc;
        const float gate = bf16_to_f32(g.HC[row * ld + f]);
        const float up = bf16_to_f32(g.HC[row * ld + g.F + f]);
        const float s = 1.0f / (1.0f + expf(-gate));
        const float silu = gate * s;
        const float dsilu = s * (1.0f + gate * (1.0f - s));
        g.out[row * ld + f] = (uint16_t)f32_to_bf16(val * up * dsilu);
        g.out[row * ld + g.F + f] = (uint16_t)f32_to_bf16(val * silu);
      }
    })
  } else {
    LRMOE_FOR_ACC({
      if (tr < rows_valid && tc < n_valid) g.out[(row0 + tr) * g.ldo + n0 + tc] = (uint16_t)f32_to_bf16(val);
    })
  }
}

// ---------------------------------------------------------------- weight-gradient kernels

struct WgradType {
  const uint16_t* A;  // [rows x M] (M contiguous)
  int64_t lda;
  const uint16_t* B;  // [rows x N] (N contiguous)
  int64_t ldb;
  float* out;         // [E x M x N]
  int M, N, ntm, ntn, tiles;
};

struct WgradArgs {
  WgradType t[2];
  int ntypes;
  int E;
  const int64_t* row_off;
  // plan (device, built by wgrad_plan_kernel): experts in decreasing chunk length
  int* plan_e;          // [E]
  int* plan_prefix;     // [E+1] items before each planned expert
  int* plan_s;          // [E] chunks of expert e (by expert id)
  int* plan_kc;         // [E] rows per chunk (multiple of BK; 0 for an empty expert)
  int64_t* plan_pbase;  // [E] first partial tile of expert e (split experts only)
  float* partials;      // [npartials x BM x BN]
  int accumulate;
};

__device__ __forceinline__ void expert_split(int64_t m, int& s, int& kc) {
  if (m <= 0) {
    s = 1;
    kc = 0;
    return;
  }
  const int64_t sc = (m + kKcMax - 1) / kKcMax;
  const int64_t per = (m + sc - 1) / sc;
  s = (int)sc;
  kc = (int)((per + BK - 1) / BK * BK);
}

// One block: order experts by decreasing chunk length (ties: lower id) and lay out items.
__global__ __launch_bounds__(NTHR) void wgrad_plan_kernel(WgradArgs g) {
  const int E = g.E;
  const int tiles = g.t[0].tiles + (g.ntypes > 1 ? g.t[1].tiles : 0);
  for (int e = threadIdx.x; e < E; e += NTHR) {
    int s, kc;
    expert_split(g.row_off[e + 1] - g.row_off[e], s, kc);
    g.plan_s[e] = s;
    g.plan_kc[e] = kc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NTHR) {
    const int kc = g.plan_kc[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int kf = g.plan_kc[f];
      rank += (kf > kc || (kf == kc && f < e)) ? 1 : 0;
    }
    g.plan_e[rank] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    int64_t pb = 0;
    for (int r = 0; r < E; ++r) {
      const int e = g.plan_e[r];
      g.plan_prefix[r] = acc;
      acc += g.plan_s[e] * tiles;
    }
    g.plan_prefix[E] = acc;
    for (int e = 0; e < E; ++e) {
      g.plan_pbase[e] = pb;
      if (g.plan_s[e] > 1) pb += (int64_t)g.plan_s[e] * tiles;
    }
  }
}

__global__ __launch_bounds__(NTHR) void wgrad_kernel(WgradArgs g) {
  __shared__ uint4 lds[2][2][kTileChunks];
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  // binary search over the planned experts
  int lo = 0, hi = g.E;  // find r with prefix[r] <= b < prefix[r+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.plan_prefix[mid] <= b) lo = mid;
    else hi = mid;
  }
  const int e = g.plan_e[lo];
  const int tiles = g.t[0].tiles + (g.ntypes > 1 ? g.t[1].tiles : 0);
  const int local = b - g.plan_prefix[lo];
  const int chunk = local / tiles, rem = local % tiles;
  const int ty = rem < g.t[0].tiles ? 0 : 1;
  const WgradType& T = g.t[ty];
  const int tile = ty == 0 ? rem : rem - g.t[0].tiles;
  const int mt = tile / T.ntn, nt = tile % T.ntn;
  const int s = g.plan_s[e], kc = g.plan_kc[e];
  const int64_t r0 = g.row_off[e], m = g.row_off[e + 1] - r0;
  const int64_t k_begin = (int64_t)chunk * kc;
  const int klen = (int)max<int64_t>(0, min<int64_t>(kc, m - k_begin));
  const int m0 = mt * BM, n0 = nt * BN;
  const int m_valid = min(BM, T.M - m0), n_valid = min(BN, T.N - n0);
  const uint16_t* Ab = T.A + (r0 + k_begin) * T.lda + m0;
  const uint16_t* Bb = T.B + (r0 + k_begin) * T.ldb + n0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[4][4];
  zero_acc(acc);
  const int nk = (klen + BK - 1) / BK;
  if (nk > 0) {
    uint4 ra[8], rb[8];
    load_mn(Ab, T.lda, m_valid, 0, klen, ra);
    load_mn(Bb, T.ldb, n_valid, 0, klen, rb);
    store_mn(lds[0][0], ra);
    store_mn(lds[0][1], rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        load_mn(Ab, T.lda, m_valid, (kt + 1) * BK, klen, ra);
        load_mn(Bb, T.ldb, n_valid, (kt + 1) * BK, klen, rb);
      }
      mma_stage(lds[cur][0], lds[cur][1], acc, wm, wn, lane);
      if (more) {
        store_mn(lds[cur ^ 1][0], ra);
        store_mn(lds[cur ^ 1][1], rb);
      }
      __syncthreads();
    }
  }
  if (s > 1) {
    float* p = g.partials + (g.plan_pbase[e] + (int64_t)chunk * tiles + rem) * (int64_t)(BM * BN);
    LRMOE_FOR_ACC({ p[tr * BN + tc] = val; })
  } else {
    float* o = T.out + (int64_t)e * T.M * T.N;
    const bool accum = g.accumulate != 0;
    LRMOE_FOR_ACC({
      if (tr < m_valid && tc < n_valid) {
        float* q = o + (int64_t)(m0 + tr) * T.N + n0 + tc;
        *q = accum ? *q + val : val;
      }
    })
  }
}

// Sums the chunk partials of every split tile in chunk order into the output.
__global__ __launch_bounds__(NTHR) void wgrad_reduce_kernel(WgradArgs g) {
  const int tiles = g.t[0].tiles + (g.ntypes > 1 ? g.t[1].tiles : 0);
  int b = blockIdx.x, e = 0;
  for (; e < g.E; ++e) {
    if (g.plan_s[e] > 1) {
      if (b < tiles) break;
      b -= tiles;
    }
  }
  if (e >= g.E) return;
  const int rem = b;
  const int ty = rem < g.t[0].tiles ? 0 : 1;
  const WgradType& T = g.t[ty];
  const int tile = ty == 0 ? rem : rem - g.t[0].tiles;
  const int m0 = (tile / T.ntn) * BM, n0 = (tile % T.ntn) * BN;
  const int m_valid = min(BM, T.M - m0), n_valid = min(BN, T.N - n0);
  const int s = g.plan_s[e];
  const float* p0 = g.partials + (g.plan_pbase[e] + rem) * (int64_t)(BM * BN);
  const int64_t pstride = (int64_t)tiles * BM * BN;
  float* o = T.out + (int64_t)e * T.M * T.N;
  for (int idx = threadIdx.x; idx < BM * BN / 4; idx += NTHR) {
    const int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
    if (r >= m_valid || c >= n_valid) continue;
    float4 sum = *(const float4*)(p0 + r * BN + c);
    for (int ch = 1; ch < s; ++ch) {
      const float4 v = *(const float4*)(p0 + ch * pstride + r * BN + c);
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    float4* q = (float4*)(o + (int64_t)(m0 + r) * T.N + n0 + c);
    if (g.accumulate) {
      const float4 old = *q;
      sum.x += old.x;
      sum.y += old.y;
      sum.z += old.z;
      sum.w += old.w;
    }
    *q = sum;
  }
}

// ---------------------------------------------------------------- f32 path

__device__ __forceinline__ int find_expert(const int64_t* row_off, int E, int64_t row) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row_off[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// out[r][n] = sum_k A[r][k] * W[e(r)][n][k]; SwiGLU epilogue or plain store.
template <int EPI>
__global__ __launch_bounds__(NTHR) void f32_dgrad_kernel(const float* __restrict__ A, int64_t lda,
                                                         const float* __restrict__ W, int64_t ldw,
                                                         int64_t w_estride, int N, int K,
                                                         const int64_t* __restrict__ row_off, int E,
                                                         const float* __restrict__ HC, float* __restrict__ out,
                                                         int64_t ldo, int F) {
  const int64_t r = blockIdx.x;
  const int n = blockIdx.y * NTHR + threadIdx.x;
  if (n >= N) return;
  const int e = find_expert(row_off, E, r);
  const float* a = A + r * lda;
  const float* w = W + (int64_t)e * w_estride + (int64_t)n * ldw;
  float acc = 0.0f;
  for (int k = 0; k < K; ++k) acc = fmaf(a[k], w[k], acc);
  if (EPI == EPI_SWIGLU) {
    const float gate = HC[r * 2 * F + n], up = HC[r * 2 * F + F + n];
    const float s = 1.0f / (1.0f + expf(-gate));
    out[r * 2 * F + n] = acc * up * (s * (1.0f + gate * (1.0f - s)));
    out[r * 2 * F + F + n] = acc * (gate * s);
  } else {
    out[r * ldo + n] = acc;
  }
}

// out[e][i][j] (+)= sum over rows r of expert e of A[r][i] * B[r][j]
__global__ __launch_bounds__(NTHR) void f32_wgrad_kernel(const float* __restrict__ A, int64_t lda,
                                                         const float* __restrict__ B, int64_t ldb, int M, int N,
                                                         const int64_t* __restrict__ row_off,
                                                         float* __restrict__ out, int accumulate) {
  const int e = blockIdx.z, i = blockIdx.y;
  const int j = blockIdx.x * NTHR + threadIdx.x;
  if (j >= N) return;
  float acc = 0.0f;
  for (int64_t r = row_off[e]; r < row_off[e + 1]; ++r) acc = fmaf(A[r * lda + i], B[r * ldb + j], acc);
  float* q = out + ((int64_t)e * M + i) * N + j;
  *q = accumulate ? *q + acc : acc;
}

// ---------------------------------------------------------------- host side

struct WgradLayout {
  size_t plan_bytes, partial_bytes;
  int64_t npartials, nitems, nreduce;
};

int wgrad_tiles(int M, int N) { return (int)(ceil_div(M, BM) * ceil_div(N, BN)); }

WgradLayout wgrad_layout(const lrmoe_problem* p, const int64_t* row_off_h) {
  const int tiles = wgrad_tiles(p->F, p->D) + (p->swiglu ? wgrad_tiles(p->D, 2 * p->F) : 0);
  WgradLayout L{};
  for (int e = 0; e < p->E; ++e) {
    const int64_t m = row_off_h[e + 1] - row_off_h[e];
    const int64_t s = m <= 0 ? 1 : ceil_div(m, kKcMax);
    L.nitems += s * tiles;
    if (s > 1) {
      L.npartials += s * tiles;
      L.nreduce += tiles;
    }
  }
  L.plan_bytes = align_up(sizeof(int) * (4 * (size_t)p->E + 1) + sizeof(int64_t) * p->E + 64, 256);
  L.partial_bytes = (size_t)L.npartials * BM * BN * sizeof(float);
  return L;
}

}  // namespace

size_t gemm_ws_bytes(const lrmoe_problem* p, const int64_t* row_off_h) {
  if (p->dtype != LRMOE_BF16) return 0;
  const WgradLayout L = wgrad_layout(p, row_off_h);
  return L.plan_bytes + L.partial_bytes;
}

lrmoe_status launch_grouped_gemm_bwd(const lrmoe_problem* p, const int64_t* row_off_h,
                                     const int64_t* row_off_d, const void* Dlt, const void* PhiC,
                                     const void* XC, const void* HC, const void* W2, const void* W1,
                                     float* dW2, float* dW1, void* dH, void* dIn, int accumulate,
                                     void* ws, hipStream_t s) {
  const int E = p->E, D = p->D, F = p->F;
  const int64_t rows = row_off_h[E];
  if (p->dtype == LRMOE_F32) {
    const float* dl = (const float*)Dlt;
    if (p->swiglu) {
      if (rows > 0) {
        f32_dgrad_kernel<EPI_SWIGLU><<<dim3((unsigned)rows, (unsigned)ceil_div(F, NTHR)), NTHR, 0, s>>>(
            dl, D, (const float*)W2, D, (int64_t)F * D, F, D, row_off_d, E, (const float*)HC, (float*)dH, 2 * F, F);
        f32_dgrad_kernel<EPI_STORE><<<dim3((unsigned)rows, (unsigned)ceil_div(D, NTHR)), NTHR, 0, s>>>(
            (const float*)dH, 2 * F, (const float*)W1, 2 * F, (int64_t)D * 2 * F, D, 2 * F, row_off_d, E, nullptr,
            (float*)dIn, D, F);
      }
      if (E > 0) {
        f32_wgrad_kernel<<<dim3((unsigned)ceil_div(D, NTHR), F, E), NTHR, 0, s>>>(
            (const float*)PhiC, F, dl, D, F, D, row_off_d, dW2, accumulate);
        f32_wgrad_kernel<<<dim3((unsigned)ceil_div(2 * F, NTHR), D, E), NTHR, 0, s>>>(
            (const float*)XC, D, (const float*)dH, 2 * F, D, 2 * F, row_off_d, dW1, accumulate);
      }
    } else {
      if (rows > 0)
        f32_dgrad_kernel<EPI_STORE><<<dim3((unsigned)rows, (unsigned)ceil_div(F, NTHR)), NTHR, 0, s>>>(
            dl, D, (const float*)W2, D, (int64_t)F * D, F, D, row_off_d, E, nullptr, (float*)dIn, F, F);
      if (E > 0)
        f32_wgrad_kernel<<<dim3((unsigned)ceil_div(D, NTHR), F, E), NTHR, 0, s>>>(
            (const float*)PhiC, F, dl, D, F, D, row_off_d, dW2, accumulate);
    }
    return launch_status();
  }

  // bf16 MFMA path
  int64_t mtiles = 0;
  for (int e = 0; e < E; ++e) mtiles += ceil_div(row_off_h[e + 1] - row_off_h[e], BM);
  DgradArgs d2{};
  d2.A = (const uint16_t*)Dlt;
  d2.lda = D;
  d2.W = (const uint16_t*)W2;
  d2.ldw = D;
  d2.w_estride = (int64_t)F * D;
  d2.N = F;
  d2.K = D;
  d2.ntn = (int)ceil_div(F, BN);
  d2.row_off = row_off_d;
  d2.E = E;
  d2.F = F;
  if (p->swiglu) {
    d2.HC = (const uint16_t*)HC;
    d2.out = (uint16_t*)dH;
    d2.ldo = 2 * F;
    if (mtiles > 0) dgrad_kernel<EPI_SWIGLU><<<(unsigned)(mtiles * d2.ntn), NTHR, 0, s>>>(d2);
    DgradArgs d1 = d2;
    d1.A = (const uint16_t*)dH;
    d1.lda = 2 * F;
    d1.W = (const uint16_t*)W1;
    d1.ldw = 2 * F;
    d1.w_estride = (int64_t)D * 2 * F;
    d1.N = D;
    d1.K = 2 * F;
    d1.ntn = (int)ceil_div(D, BN);
    d1.HC = nullptr;
    d1.out = (uint16_t*)dIn;
    d1.ldo = D;
    if (mtiles > 0) dgrad_kernel<EPI_STORE><<<(unsigned)(mtiles * d1.ntn), NTHR, 0, s>>>(d1);
  } else {
    d2.out = (uint16_t*)dIn;
    d2.ldo = F;
    if (mtiles > 0) dgrad_kernel<EPI_STORE><<<(unsigned)(mtiles * d2.ntn), NTHR, 0, s>>>(d2);
  }

  const WgradLayout L = wgrad_layout(p, row_off_h);
  WgradArgs w{};
  w.t[0] = WgradType{(const uint16_t*)PhiC, F, (const uint16_t*)Dlt, D, dW2, F, D,
                     (int)ceil_div(F, BM), (int)ceil_div(D, BN), wgrad_tiles(F, D)};
  w.ntypes = 1;
  if (p->swiglu) {
    w.t[1] = WgradType{(const uint16_t*)XC, D, (const uint16_t*)dH, 2 * F, dW1, D, 2 * F,
                       (int)ceil_div(D, BM), (int)ceil_div(2 * F, BN), wgrad_tiles(D, 2 * F)};
    w.ntypes = 2;
  }
  w.E = E;
  w.row_off = row_off_d;
  char* b = (char*)ws;
  w.plan_e = (int*)b;
  w.plan_prefix = w.plan_e + E;
  w.plan_s = w.plan_prefix + E + 1;
  w.plan_kc = w.plan_s + E;
  w.plan_pbase = (int64_t*)(b + align_up(sizeof(int) * (4 * (size_t)E + 1), 8));
  w.partials = (float*)(b + L.plan_bytes);
  w.accumulate = accumulate;
  if (E > 0) {
    wgrad_plan_kernel<<<1, NTHR, 0, s>>>(w);
    wgrad_kernel<<<(unsigned)L.nitems, NTHR, 0, s>>>(w);
    if (L.nreduce > 0) wgrad_reduce_kernel<<<(unsigned)L.nreduce, NTHR, 0, s>>>(w);
  }
  return launch_status();
}

}  // namespace lrmoe
