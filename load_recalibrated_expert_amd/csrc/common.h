// Internal helpers shared by the HIP kernels of liblrmoe (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrmoe.h"

namespace lrmoe {

constexpr int kWave = 64;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of data read once (streamed past the caches' retention policy).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 (lo in bits 0..15), round to nearest, ties to even, with gfx950's
// v_cvt_pk_bf16_f32: one instruction per pair. For finite inputs (denormals, ties, overflow to
// infinity included) it gives the same bits as adding 0x7FFF plus the kept lsb and truncating.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// bf16 nearest (ties to even) of the *exact* product a*b, for a, b finite floats whose
// exact product fits 48 bits (a f32 times a bf16 value). p = fl(a*b) can only land on the
// other side of a bf16 rounding boundary by becoming the boundary itself (the midpoint is
// an f32 value), so only that case consults the exact error e = a*b - p from the FMA.
__device__ __forceinline__ uint32_t mul_to_bf16(float a, float b) {
  float p = a * b;
  float e = __builtin_fmaf(a, b, -p);
  uint32_t u = __float_as_uint(p);
  uint32_t lo = u & 0xFFFFu;
  uint32_t hi = u >> 16;
  if (lo > 0x8000u) {
    hi += 1u;
  } else if (lo == 0x8000u) {
    if (e == 0.0f) hi += (hi & 1u);
    else if ((e > 0.0f) == (p > 0.0f)) hi += 1u;
  }
  return hi & 0xFFFFu;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum of squares of 8 bf16 values held in a uint4, in fp64 (each square is exact).
__device__ __forceinline__ double sumsq_bf16x8(uint4 v) {
  double s = 0.0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
    s += (double)(a * a);
    s += (double)(b * b);
  }
  return s;
}
// Sum of magnitudes of 8 bf16 values held in a uint4, in fp64.
__device__ __forceinline__ double sumabs_bf16x8(uint4 v) {
  double s = 0.0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += (double)fabsf(bf16_lo(w[i]));
    s += (double)fabsf(bf16_hi(w[i]));
  }
  return s;
}
// Sum of magnitudes of 4 floats held in a uint4, in fp64.
__device__ __forceinline__ double sumabs_f32x4(uint4 v) {
  return (double)fabsf(__uint_as_float(v.x)) + (double)fabsf(__uint_as_float(v.y)) +
         (double)fabsf(__uint_as_float(v.z)) + (double)fabsf(__uint_as_float(v.w));
}
// Sum of squares of 4 floats held in a uint4, in fp64.
__device__ __forceinline__ double sumsq_f32x4(uint4 v) {
  double a = __uint_as_float(v.x), b = __uint_as_float(v.y), c = __uint_as_float(v.z),
         d = __uint_as_float(v.w);
  return a * a + b * b + c * c + d * d;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline lrmoe_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? LRMOE_OK : LRMOE_ERR_HIP;
}

// ---------------------------------------------------------------- launchers (one per .hip file)

lrmoe_status launch_score(const lrmoe_problem* p, const void* G, const void* Phi, const float* alpha,
                          const int32_t* tok, float* R, double* gn, hipStream_t s);
lrmoe_status launch_score_gradient(const lrmoe_problem* p, bool magnitude, const void* G, const int32_t* tok,
                                    float* R, double* gs, hipStream_t s);

size_t select_ws_bytes(const lrmoe_problem* p);
lrmoe_status launch_select(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                           const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel,
                           uint8_t* keep, const int32_t* tok, const int32_t* slot, int32_t* pmap,
                           int32_t* ctok, int32_t* cslot, void* ws, hipStream_t s);

size_t select_noalloc_max_bytes();
lrmoe_status launch_select_noalloc(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                                   const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel, uint8_t* keep,
                                   const int32_t* tok, const int32_t* slot, int32_t* pmap, int32_t* ctok,
                                   int32_t* cslot, hipStream_t s);

lrmoe_status launch_compact(const lrmoe_problem* p, int64_t rows, bool masked, const int32_t* sel,
                            const uint8_t* keep, const void* G, const void* Phi, const void* X,
                            const void* H, const float* alpha, const int32_t* tok, const int32_t* slot,
                            void* Dlt, void* PhiC, void* XC, void* HC, int32_t* ctok, int32_t* cslot,
                            const int32_t* pmap, void* ws, hipStream_t s);
size_t compact_ws_bytes(const lrmoe_problem* p);
lrmoe_status launch_compact_weighted_phi(const lrmoe_problem* p, int64_t rows, const int32_t* sel,
                                         const void* Phi, const float* alpha, void* PhiW, hipStream_t s);

lrmoe_status launch_expert_forward(const lrmoe_problem* p, const int64_t* seg_off_d, const void* X,
                                   const int32_t* tok, const float* alpha, const void* W1, const void* W2, void* H,
                                   void* Phi, void* Y, hipStream_t s);
size_t gemm_ws_bytes(const lrmoe_problem* p, const int64_t* row_off_h);
lrmoe_status launch_grouped_gemm_bwd(const lrmoe_problem* p, const int64_t* row_off_h,
                                     const int64_t* row_off_d, const void* Dlt, const void* PhiC,
                                     const void* XC, const void* HC, const int32_t* hc_rows,
                                     const int32_t* phi_rows, const int32_t* x_rows, const int32_t* dlt_rows,
                                     const float* alpha, const void* W2, const void* W1,
                                     float* dW2, float* dW1, void* dH, void* dIn, int accumulate,
                                     void* ws, hipStream_t s, hipEvent_t din_ready);

size_t scatter_ws_bytes(const lrmoe_problem* p);
lrmoe_status launch_scatter(const lrmoe_problem* p, int mode, int64_t n_rows, int width, int rows_dtype,
                            const void* rows, const int32_t* ctok, const int32_t* cslot, const int32_t* pmap,
                            float* out, void* ws, hipStream_t s);

}  // namespace lrmoe
