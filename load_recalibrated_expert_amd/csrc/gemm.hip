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
// Without a packed Dlt = alpha g (the path that reads gradient rows by token), the FC2
// products take the routing weight elsewhere, which the weight gradient's bilinearity
// allows (appendix 7.1, Eq. 6-8): the data gradient reads the token rows g[ctok] and
// scales each fp32 row of g W2^T by its pair's alpha before the SwiGLU backward, and the
// weight gradient reads the weighted saved rows PhiW = alpha Phi as A and g[ctok] as B.
// Any operand can be read in place through a row map instead of packed (a mapped row
// outside its matrix reads as zeros).
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulation. A block of 512 threads
// (eight 64-wide wavefronts, two per SIMD) owns a 256x256 output tile; each wavefront a
// 128x64 sub-tile held as 2x4 MFMA accumulators. K advances 32 per stage through four LDS
// stages (4 x 32 KB) filled by direct global-to-LDS loads issued three stages ahead, one
// barrier per stage; the data gradients instead run two 64-K stages in the same 128 KB, so
// each request of their K-contiguous operands is a whole 128-byte line. Finished tiles
// leave through LDS so every output row is written by
// consecutive threads with 16-byte accesses. Weight-gradient tiles split the packed rows
// of large experts into K chunks; chunk partials go to the workspace and a second kernel
// sums them in chunk order, so results do not depend on scheduling. Tiles are handed to
// the 8 XCDs (hardware round-robins blocks over them) in contiguous runs, so tiles that
// share operand panels meet in one L2; weight-gradient runs are cut by work, not count.
//
// f32 path (small problems): plain fp32 FMA kernels, no bf16 anywhere.
#include <algorithm>
#include <functional>
#include <mutex>
#include <vector>

#include "common.h"

namespace lrmoe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int BM = 256, BK = 32;
// Block tile configuration: a 256 x BN output tile per block on a 2 x WN grid of
// wavefronts; each wavefront owns a 128 x (BN / WN) sub-tile held as MB x NB MFMA
// accumulators of 32 x 32. Eight wavefronts (two per SIMD) hold 128 x 64 sub-tiles in 128
// VGPRs each; four wavefronts (one per SIMD) hold 128 x 128 sub-tiles in 256 accumulation
// registers, which reads a third fewer LDS bytes per MFMA. K advances 32 per stage through
// STAGES LDS stages of 32 KB. (Two blocks of 4 wavefronts per CU with 256 x 128 tiles and
// three 24 KB stages each, so that one block's epilogue overlaps the other's MFMAs, ran the
// data gradients 7% slower: with one stage less, each direct load has a single K step to land.)
template <int NWAVE_, int BN_, int STAGES_>
struct TileCfg {
  static constexpr int NWAVE = NWAVE_, NTHR = NWAVE_ * 64, BN = BN_, STAGES = STAGES_;
  static constexpr int WM = 2, WN = NWAVE_ / 2;  // wave grid over the tile (M x N)
  static constexpr int MB = BM / WM / 32, NB = BN_ / WN / 32;  // 32-wide MFMA blocks per wavefront
  static constexpr int NL = BM * BK * 2 / 1024 / NWAVE_;  // 1 KB direct loads per wave per 256-row operand
  static constexpr int A_U4 = BM * BK * 2 / 16, B_U4 = BN_ * BK * 2 / 16;  // uint4 per stage
  static_assert(WN * NB * 32 == BN_ && WM * MB * 32 == BM, "wave tiles cover the block tile");
};
using CfgW = TileCfg<8, 256, 4>;  // weight gradients and the forward
using CfgD = TileCfg<8, 256, 4>;  // data gradients
// the weight-gradient configuration, also used by the host side
constexpr int BN = CfgW::BN, STAGES = CfgW::STAGES;
// threads of the small kernels (plan, split-K reduction, f32 path)
constexpr int kAuxThr = 512;
// Candidate lengths (packed rows) of a weight-gradient chunk, the longest first; the host
// picks one per problem (wgrad_schedule)
constexpr int64_t kKcCandidates[] = {12288, 8192, 6144};
constexpr uint32_t kOOB = 0x80000000u;     // buffer offset past num_records: the load returns 0

// Kernel attributes of a block of C::NWAVE wavefronts: with one wavefront per SIMD the
// wavefront may hold 512 registers (256 of them accumulation registers).
#define LRMOE_GEMM_ATTR(C) __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::NWAVE / 4, C::NWAVE / 4)))

__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, i = b >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + i;
}

// Raw buffer resource over [p, p + 2 GiB): loads at offsets >= 2^31 return zeros without
// touching memory, which is how tile edges are masked without branches.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7FFFFFFF, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// lds_wave_base + 16 l (lds_wave_base is wave-uniform). Out-of-range offsets write zeros.
__device__ __forceinline__ void dma16(rsrc_t r, const uint4* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds_wave_base), 16, off, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS layouts
//
// K-contiguous operand in 32-K stages (the forward's A operand; the data gradients use the
// 64-K stages further down): a stage holds R rows (256 or 128) x 32 K values
// (64 bytes per row, four 16-byte chunks). Rows 2L and 2L + 1 share the 128-byte LDS line L,
// which holds eight 16-byte slots: chunk c of row 2L + h sits in slot (4 h + c) ^ ((L / 2) % 4).
// The LDS has 64 four-byte banks and serves a 16-byte read 16 lanes at a time. An MFMA
// fragment read gives lane i one chunk of row row0 + i (row0 a multiple of 32), so each group
// of 16 lanes reads 8 lines, two rows per line: the line's parity picks one half of the banks
// and h with (L / 2) % 4 picks 8 distinct slots per half, so the 16 lanes hit all 64 banks.
// (Pairing rows r and r + R/2 with the swizzle L % 8 covered 32 banks per 8 lanes, a two-way
// conflict on every read: half the LDS cycles of the data gradients went to conflicts.)
//
// Row-major-in-K operand (weight-gradient GEMMs): a stage holds 32 K rows x 256 columns,
// 512 bytes per row as eight 64-byte segments; segment s of row k sits in slot s ^ (k & 3),
// so the 4-row transpose reads of one half-wavefront cover all 64 banks.

template <class C>
struct StageBufs {
  uint4 a[C::STAGES][C::A_U4];
  uint4 b[C::STAGES][C::B_U4];
};

// uint4 index of chunk c of row r in a K-contiguous stage
__device__ __forceinline__ int nt_slot(int r, int c) {
  const int line = r >> 1;
  return line * 8 + ((((r & 1) << 2) | c) ^ ((line >> 1) & 3));
}

// Direct-to-LDS loader of a K-contiguous operand of ROWS rows per stage, for blocks of
// NWAVE wavefronts. A 1 KB direct load fills 8 LDS lines (16 tile rows); wave w issues
// loads j = 0..NL-1 covering lines 8 (w*NL + j) + l/8, and lane l fetches the chunk that
// belongs in slot l % 8 of its line: with x = (l % 8) ^ ((line / 2) % 4), that is chunk x % 4
// of row 2 line + x / 4. Since 8 divides the first line of a load, (line / 2) % 4 = (l / 16) % 4
// and the lane's chunk is the same in every load.
template <int NWAVE_, int ROWS>
struct DmaK {
  static constexpr int NL = ROWS / 16 / NWAVE_;  // direct loads per wavefront
  static_assert(NL * 16 * NWAVE_ == ROWS, "whole loads per wavefront");
  rsrc_t r;
  uint32_t off[NL];
  int col;    // first K element of this lane's chunk within the stage
  int wbase;  // uint4 offset of this wave's region in a stage
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld, int rows_valid) {
    r = make_rsrc(p);
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int logical = (l & 7) ^ ((l >> 4) & 3);
    col = (logical & 3) * 8;
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int row = 2 * ((w * NL + j) * 8 + (l >> 3)) + (logical >> 2);
      off[j] = row < rows_valid ? (uint32_t)((row * ld + col) * 2) : kOOB;
    }
  }
  // Tile row r is row rows[r] of the matrix at p (its rows are gathered; a mapped row outside
  // [0, nrows) reads as zeros). The rows stay fixed along K, so the map is read once here.
  // The byte offsets are 32-bit: the host keeps nrows * ld * 2 under 2 GiB.
  __device__ __forceinline__ void init_rows(const uint16_t* p, int64_t ld, int rows_valid, const int32_t* rows,
                                            int64_t nrows) {
    r = make_rsrc(p);
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int logical = (l & 7) ^ ((l >> 4) & 3);
    col = (logical & 3) * 8;
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int row = 2 * ((w * NL + j) * 8 + (l >> 3)) + (logical >> 2);
      const int64_t src = row < rows_valid ? (int64_t)rows[row] : -1;
      off[j] = (src >= 0 && src < nrows) ? (uint32_t)((src * ld + col) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ void issue_one(int j, const uint4* stage, int k0, int kend, uint32_t) const {
    const bool kok = k0 + col < kend;
    dma16(r, stage + wbase + j * 64, (kok && off[j] != kOOB) ? off[j] + (uint32_t)k0 * 2u : kOOB);
  }
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void fetch(int) {}
  __device__ __forceinline__ void advance(int) {}
};

// Direct-to-LDS loader of a row-major-in-K operand, NL_ 1 KB loads per wavefront per stage.
// A 1 KB direct load fills 2 K rows; wave w issues loads j covering rows 2 (w*NL + j) + l/32,
// and lane l fetches the chunk that belongs in 16-byte slot l % 32 of its row.
template <int NL_>
struct DmaT {
  static constexpr int NL = NL_;
  rsrc_t r;
  uint32_t off[NL];
  int row[NL];
  int wbase;
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld, int mn_valid) {
    r = make_rsrc(p);
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int k = (w * NL + j) * 2 + (l >> 5);
      const int pc = l & 31;
      const int c = (((pc >> 2) ^ (k & 3)) << 2) | (pc & 3);  // logical 16-byte chunk
      row[j] = k;
      off[j] = c * 8 < mn_valid ? (uint32_t)((k * ld + c * 8) * 2) : kOOB;
    }
  }
  // SwiGLU pairing of a [K x 2F] weight: tile columns 0..127 are the gate columns j0..j0+127
  // and tile columns 128..255 the matching up columns F+j0..F+j0+127; columns at or past F
  // in either half read as zeros.
  __device__ __forceinline__ void init_paired(const uint16_t* p, int64_t ld, int j0, int F) {
    r = make_rsrc(p);
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int k = (w * NL + j) * 2 + (l >> 5);
      const int pc = l & 31;
      const int c = (((pc >> 2) ^ (k & 3)) << 2) | (pc & 3);  // logical 16-byte chunk
      const int t = c * 8;                                     // tile column
      const int f = t < 128 ? j0 + t : j0 + t - 128;           // column within its half
      const int64_t src = t < 128 ? f : (int64_t)F + f;
      row[j] = k;
      off[j] = f < F ? (uint32_t)((k * ld + src) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ void issue_one(int j, const uint4* stage, int k0, int kend, uint32_t kstep) const {
    dma16(r, stage + wbase + j * 64, (off[j] != kOOB && k0 + row[j] < kend) ? off[j] + (uint32_t)k0 * kstep : kOOB);
  }
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void fetch(int) {}
  __device__ __forceinline__ void advance(int) {}
};

typedef __attribute__((address_space(4))) const int32_t const_i32_t;

// The same operand with gathered K rows: K row k of the item is row idx[k] of the matrix
// (saved activations read in place instead of packed). A lane's 16-byte chunk sits at
// row * pitch + its column offset, so the buffer resource spans the whole matrix (under
// 2 GiB; the host checks). Rows outside [0, nrows) read as zeros. A wavefront needs 2 NL row
// indices per stage, rows 2 (w NL + j) + h for its loads j < NL and halves h = 0, 1. It reads
// them with scalar loads (the index array is constant during the kernel), issued at the top
// of the loop iteration whose end turns them into the load offsets of a later stage. Scalar
// loads are not counted by the vector-memory counter whose fixed counts the K loop waits
// on, and the wait for them falls together with the loop's wait for its own LDS reads.
// Reads are clamped to [0, klen) so they never leave the item's part of the index array.
template <int NL_>
struct DmaTG {
  static constexpr int NL = NL_;
  rsrc_t r;                        // the matrix
  const_i32_t* idx;                // the item's row indices
  uint32_t coff[NL];               // column offset in bytes, or kOOB past the tile's columns
  int row[NL];                     // K row within a stage
  int wbase, w, h;
  uint32_t pitch, nrows;
  int klen;
  int32_t e[2 * NL];               // indices of rows 2 w NL .. 2 w NL + 2 NL - 1 of the stage being prepared
  uint32_t off[NL];                // byte offsets of the stage to issue next (kOOB: zeros)
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld, int mn_valid, const int32_t* idx_, int klen_,
                                       int64_t nrows_) {
    r = make_rsrc(p);
    idx = (const_i32_t*)idx_;
    klen = klen_;
    nrows = (uint32_t)nrows_;
    pitch = (uint32_t)(ld * 2);
    const int lane = threadIdx.x & 63;
    w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    h = lane >> 5;
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int k = (w * NL + j) * 2 + h;
      const int pc = lane & 31;
      const int c = (((pc >> 2) ^ (k & 3)) << 2) | (pc & 3);
      row[j] = k;
      coff[j] = c * 8 < mn_valid ? (uint32_t)(c * 8 * 2) : kOOB;
      off[j] = kOOB;
    }
  }
  __device__ __forceinline__ void load_indices(int s) {
#pragma unroll
    for (int i = 0; i < 2 * NL; ++i) e[i] = idx[min(s * BK + 2 * NL * w + i, klen - 1)];
  }
  __device__ __forceinline__ void start() {
    load_indices(0);
    advance(0);
  }
  // the indices of stage s (scalar loads; advance(s) turns them into load offsets)
  __device__ __forceinline__ void fetch(int s) { load_indices(s); }
  // stage s's load offsets from its indices (loaded by fetch(s)), computed ahead, where the
  // wavefront waits anyway, so that issuing the loads costs no arithmetic
  __device__ __forceinline__ void advance(int s) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int32_t mrow = h ? e[2 * j + 1] : e[2 * j];
      const bool ok = s * BK + row[j] < klen && (uint32_t)mrow < nrows && coff[j] != kOOB;
      off[j] = ok ? (uint32_t)mrow * pitch + coff[j] : kOOB;
    }
  }
  __device__ __forceinline__ void issue_one(int j, const uint4* stage, int, int, uint32_t) const {
    dma16(r, stage + wbase + j * 64, off[j]);
  }
};

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

// MFMA fragment (32 columns from `col0`, 16 reduction rows from `k0`) out of a row-major-in-K
// stage with the gfx950 LDS transpose read. Within each 16-lane group the read hands lane
// i the (i%4)-th 16-bit element of the 8-byte segments addressed by lanes i/4, i/4+4,
// i/4+8, i/4+12 of the group. So lane s of group g addresses reduction row
// k0 + 8*(g/2) + s/4 at columns col0 + 16*(g%2) + 4*(s%4): lane i then holds column
// col0 + 16*(g%2) + i at 4 consecutive reduction rows, and two reads (rows +0..3, +4..7)
// give the 8 consecutive K values of the MFMA operand layout.
__device__ __forceinline__ bf16x8_t frag_tr(const uint4* stage, int col0, int k0, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int k = k0 + 8 * (g >> 1) + (sl >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (sl & 3);
  const int pcol = ((((col >> 5) ^ (k & 3))) << 5) | (col & 31);  // rows k and k+4 share k & 3
  const __attribute__((address_space(3))) short* base =
      (const __attribute__((address_space(3))) short*)(const lds_void_t*)stage;
  const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + k * BM + pcol));
  const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + (k + 4) * BM + pcol));
  typedef short v8s_t __attribute__((ext_vector_type(8)));
  const v8s_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, both);
}

// ---------------------------------------------------------------- MFMA on one LDS stage

// la holds the 256 output rows' operand (m), lb the 256 output columns' operand (n).
// The MFMA takes the n fragment first, so each lane's accumulator holds 4 consecutive
// output columns of one output row: acc[nb][mb][v] is output row
// wm*(32 MB) + mb*32 + lane%32, column wn*(32 NB) + nb*32 + 8*(v/4) + 4*(lane/32) + v%4.
// One MFMA fragment: rows row0..row0+31 of an operand stage, K16 step kk.
template <bool TN>
__device__ __forceinline__ bf16x8_t load_frag(const uint4* __restrict__ stage, int row0, int kk, int lane) {
  if constexpr (TN) {
    return frag_tr(stage, row0, kk * 16, lane);
  } else {
    return __builtin_bit_cast(bf16x8_t, stage[nt_slot(row0 + (lane & 31), kk * 2 + (lane >> 5))]);
  }
}

template <class C>
using acc_t = f32x16_t[C::NB][C::MB];

template <class C>
__device__ __forceinline__ void zero_acc(acc_t<C>& acc) {
#pragma unroll
  for (int i = 0; i < C::NB; ++i)
#pragma unroll
    for (int j = 0; j < C::MB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
}

__device__ __forceinline__ void mfma(f32x16_t& acc, const bf16x8_t& n_frag, const bf16x8_t& m_frag) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(n_frag, m_frag, acc, 0, 0, 0);
}

// The K loop shared by every bf16 GEMM. S = C::STAGES LDS stages of 32 K values per operand
// are filled by direct loads issued S-1 stages ahead. At the top of stage kt each wave waits
// for its own loads of stage kt+1, and one barrier then makes stage kt+1 visible and frees
// stage kt-1's buffer, into which stage kt+S-1 is loaded. A stage is two K16 steps of
// NB x MB MFMAs. The wavefront issues in order, so every memory instruction sits right
// behind an MFMA (hard scheduling fences keep that order): during the first step the
// direct loads of stage kt+S-1 and the fragments of the second step; during the
// second step the fragments of stage kt+1's first step, so MFMAs start right after the next
// barrier. With 16 MFMAs per step the fragment reads take the first slots and the direct
// loads the following ones; with 8 they share the first slots.
template <class C, bool TNA, bool TNB, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(StageBufs<C>& sm, LA& la, LB& lb, int kend, uint32_t kstep_a,
                                              uint32_t kstep_b, acc_t<C>& acc, int wm, int wn, int lane) {
  constexpr int MB = C::MB, NB = C::NB;
  constexpr int NM = NB * MB, STAGES = C::STAGES, NLA = LA::NL, NLB = LB::NL;
  // first MFMA slot of the direct loads: behind the fragment reads when the step has room
  // for both, else from the first slot on, beside them
  constexpr int kDma0 = NM >= MB + NB + NLA + NLB ? MB + NB : 0;
  static_assert(NLA + NLB <= NM, "one direct load per MFMA slot of the first K16 step");
  const int nk = (kend + BK - 1) / BK;
  if (nk <= 0) return;
  la.start();
  lb.start();
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
#pragma unroll
    for (int j = 0; j < (NLA > NLB ? NLA : NLB); ++j) {
      if (j < NLA) la.issue_one(j, sm.a[s], s * BK, kend, kstep_a);
      if (j < NLB) lb.issue_one(j, sm.b[s], s * BK, kend, kstep_b);
    }
    la.fetch(s + 1);  // the indices of stage s + 1
    lb.fetch(s + 1);
    la.advance(s + 1);
    lb.advance(s + 1);
  }
  // stage 0 landed: the loads of stages 1..STAGES-2 may still be in flight (every stage
  // issues NLA + NLB direct loads per wavefront and nothing else on this counter)
  constexpr int kPro = (STAGES - 2) * (NLA + NLB), kLoop = (STAGES - 3) * (NLA + NLB);
  static_assert(kPro < 64 && kLoop >= 0, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kPro & 0xF) | ((kPro >> 4) << 14));
  __syncthreads();
  bf16x8_t fa[2][MB], fb[2][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) fa[0][i] = load_frag<TNA>(sm.a[0], wm * 32 * MB + i * 32, 0, lane);
#pragma unroll
  for (int i = 0; i < NB; ++i) fb[0][i] = load_frag<TNB>(sm.b[0], wn * 32 * NB + i * 32, 0, lane);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt % STAGES, nxt = (kt + 1) % STAGES, ldst = (kt + STAGES - 1) % STAGES;
    const int k_ld = (kt + STAGES - 1) * BK;
    // stage kt+1 landed: the loads of stages kt+2..kt+STAGES-2 may still be in flight
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoop & 0xF) | ((kLoop >> 4) << 14));
    __syncthreads();
    la.fetch(kt + STAGES);
    lb.fetch(kt + STAGES);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      mfma(acc[i / MB][i % MB], fb[0][i / MB], fa[0][i % MB]);
      __builtin_amdgcn_sched_barrier(0);
      if (i >= kDma0 && i < kDma0 + NLA) la.issue_one(i - kDma0, sm.a[ldst], k_ld, kend, kstep_a);
      else if (i >= kDma0 + NLA && i < kDma0 + NLA + NLB)
        lb.issue_one(i - kDma0 - NLA, sm.b[ldst], k_ld, kend, kstep_b);
      if (i < MB) fa[1][i] = load_frag<TNA>(sm.a[cur], wm * 32 * MB + i * 32, 1, lane);
      else if (i < MB + NB) fb[1][i - MB] = load_frag<TNB>(sm.b[cur], wn * 32 * NB + (i - MB) * 32, 1, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      mfma(acc[i / MB][i % MB], fb[1][i / MB], fa[1][i % MB]);
      __builtin_amdgcn_sched_barrier(0);
      if (i < MB) fa[0][i] = load_frag<TNA>(sm.a[nxt], wm * 32 * MB + i * 32, 0, lane);
      else if (i < MB + NB) fb[0][i - MB] = load_frag<TNB>(sm.b[nxt], wn * 32 * NB + (i - MB) * 32, 0, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    la.advance(kt + STAGES);
    lb.advance(kt + STAGES);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the loop
}

// ---------------------------------------------------------------- data-gradient K loop, 64-K stages
//
// Both data-gradient operands are contiguous along K. In a 32-K stage a row contributes 64
// bytes, so every request of the direct loads is half a 128-byte line. In a 64-K stage row
// r fills LDS line r and eight consecutive lanes fetch it, so each request is a whole line.
// Two such stages of both 256-row operands take the same 128 KB as four 32-K stages. Chunk c
// (K values 8c..8c+7) of row r sits in 16-byte slot c ^ ((r / 2) % 8) of line r: the 8 even
// rows among 16 consecutive ones then take 8 distinct slots in one half of the 64 banks and
// the 8 odd rows in the other, so a 16-lane fragment read is free of bank conflicts.
constexpr int BK64 = 64;

template <int NWAVE_, int ROWS>
struct DmaK64 {
  static constexpr int NL = ROWS / 8 / NWAVE_;  // 1 KB direct loads (8 rows) per wavefront per stage
  static_assert(NL * 8 * NWAVE_ == ROWS, "whole loads per wavefront");
  rsrc_t r;
  uint32_t off[NL];
  int col[NL];  // first K element of this lane's chunk in load j (it depends on the load's row)
  int wbase;
  // the row and chunk of lane l in load j: row 8 (w NL + j) + l/8, chunk (l % 8) ^ ((row / 2) % 8)
  __device__ __forceinline__ static int lane_row(int w, int j, int l) { return 8 * (w * NL + j) + (l >> 3); }
  __device__ __forceinline__ static int lane_chunk(int row, int l) { return (l & 7) ^ ((row >> 1) & 7); }
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld, int rows_valid) {
    r = make_rsrc(p);
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int row = lane_row(w, j, l);
      col[j] = lane_chunk(row, l) * 8;
      off[j] = row < rows_valid ? (uint32_t)((row * ld + col[j]) * 2) : kOOB;
    }
  }
  // tile row r is row rows[r] of the matrix at p, as DmaK::init_rows
  __device__ __forceinline__ void init_rows(const uint16_t* p, int64_t ld, int rows_valid, const int32_t* rows,
                                            int64_t nrows) {
    r = make_rsrc(p);
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wbase = w * NL * 64;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int row = lane_row(w, j, l);
      col[j] = lane_chunk(row, l) * 8;
      const int64_t src = row < rows_valid ? (int64_t)rows[row] : -1;
      off[j] = (src >= 0 && src < nrows) ? (uint32_t)((src * ld + col[j]) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ void issue_one(int j, const uint4* stage, int k0, int kend) const {
    dma16(r, stage + wbase + j * 64, (off[j] != kOOB && k0 + col[j] < kend) ? off[j] + (uint32_t)k0 * 2u : kOOB);
  }
};

// two 64-K stages of both 256-row operands, in the same bytes as StageBufs<CfgD>
struct StageBufs64 {
  uint4 a[2][BM * BK64 * 2 / 16];
  uint4 b[2][BM * BK64 * 2 / 16];
};

__device__ __forceinline__ bf16x8_t load_frag64(const uint4* __restrict__ stage, int row0, int kk, int lane) {
  const int r = row0 + (lane & 31), c = kk * 2 + (lane >> 5);
  return __builtin_bit_cast(bf16x8_t, stage[r * 8 + (c ^ ((r >> 1) & 7))]);
}

// Two stages of 64 K values per operand, 4 K16 steps of NB x MB MFMAs each. Iteration kt:
//   steps 0-2: MFMAs of stage kt, each step reading the next step's fragments behind them;
//   wait for this wavefront's loads of stage kt+1 and its fragment reads, one barrier: stage
//     kt+1 is visible, and every wavefront holds its fragments of stage kt in registers;
//   step 3: MFMAs of stage kt's last step; the direct loads of stage kt+2 into stage kt's
//     buffer (B's before A's: 0.9-1.5% faster in the FC1 data gradient than A's first), and
//     the fragments of stage kt+1's first step (in the last iterations the loads are past
//     kend and write zeros, and the fragments go unused).
// A stage's loads thus have four K16 steps to land, as in the 32-K loop, with one barrier per
// 64 K instead of two, and the wait is for every load in flight (vmcnt 0), not a count.
// (A third stage of A in all 160 KB of LDS, its loads left in flight at the wait, measured
// about 1% slower.)
template <class C, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop_k64(StageBufs64& sm, LA& la, LB& lb, int kend, acc_t<C>& acc,
                                                  int wm, int wn, int lane) {
  constexpr int MB = C::MB, NB = C::NB, NM = NB * MB, NLA = LA::NL, NLB = LB::NL;
  static_assert(C::BN == BM && sizeof(StageBufs64) <= sizeof(StageBufs<C>), "two stages of both operands fit");
  static_assert(NLA + NLB <= 2 * NM, "at most two direct loads per MFMA slot of step 3");
  const int nk = (kend + BK64 - 1) / BK64;
  if (nk <= 0) return;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int j = 0; j < NLB; ++j) lb.issue_one(j, sm.b[s], s * BK64, kend);
#pragma unroll
    for (int j = 0; j < NLA; ++j) la.issue_one(j, sm.a[s], s * BK64, kend);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  bf16x8_t fa[2][MB], fb[2][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) fa[0][i] = load_frag64(sm.a[0], wm * 32 * MB + i * 32, 0, lane);
#pragma unroll
  for (int i = 0; i < NB; ++i) fb[0][i] = load_frag64(sm.b[0], wn * 32 * NB + i * 32, 0, lane);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    const int k_ld = (kt + 2) * BK64;  // at or past kend in the last two iterations: zeros
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      const int h = st & 1;  // fragments in use: fa[h], fb[h]; the next step's go to fa[h ^ 1]
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        mfma(acc[i / MB][i % MB], fb[h][i / MB], fa[h][i % MB]);
        __builtin_amdgcn_sched_barrier(0);
        if (i < MB) fa[h ^ 1][i] = load_frag64(sm.a[cur], wm * 32 * MB + i * 32, st + 1, lane);
        else if (i < MB + NB) fb[h ^ 1][i - MB] = load_frag64(sm.b[cur], wn * 32 * NB + (i - MB) * 32, st + 1, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // vmcnt(0) lgkmcnt(0): this wavefront's loads of stage kt+1 landed and its reads of stage
    // kt's last fragments returned, so after the barrier stage kt's buffer may be refilled
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      mfma(acc[i / MB][i % MB], fb[1][i / MB], fa[1][i % MB]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 2 * i + u;
        if (j < NLB) lb.issue_one(j, sm.b[cur], k_ld, kend);
        else if (j < NLA + NLB) la.issue_one(j - NLB, sm.a[cur], k_ld, kend);
      }
      if (i < MB) fa[0][i] = load_frag64(sm.a[nxt], wm * 32 * MB + i * 32, 0, lane);
      else if (i < MB + NB) fb[0][i - MB] = load_frag64(sm.b[nxt], wn * 32 * NB + (i - MB) * 32, 0, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the loop
}

// ---------------------------------------------------------------- epilogue through LDS

// Writes the accumulators out through LDS so that every output row is handled by
// consecutive threads with 16-byte accesses. The 256 x BN fp32 tile is staged in two halves
// of 128 rows (the wavefronts with wm = 0, then wm = 1), each filling the stage buffers
// (128 x 256 x 4 = 128 KB, all four stages). A staged row holds BN/4 chunks of 4 floats;
// chunk c of row r sits in slot c ^ (r & 15), so the accumulator writes (32 rows per
// instruction) and the row reads both spread over the banks.
template <class C>
__device__ __forceinline__ void stage_half(float4* st, const acc_t<C>& acc, int wn, int lane) {
  constexpr int P = C::BN / 4;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = mb * 32 + (lane & 31);
        const int c = (wn * 32 * C::NB + nb * 32 + 8 * q + 4 * (lane >> 5)) >> 2;
        st[r * P + (c ^ (r & 15))] =
            make_float4(acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1], acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]);
      }
}

// BODY(row, col, v[8]) receives 8 consecutive columns of one tile row.
template <class C, class Body>
__device__ __forceinline__ void epilogue_staged(StageBufs<C>& sm, const acc_t<C>& acc, int wm, int wn, int lane,
                                                Body body) {
  constexpr int P = C::BN / 4, NT = C::NTHR;
  static_assert((BM / 2) * C::BN * 4 <= (int)sizeof(StageBufs<C>), "a staged half fits the stage buffers");
  float4* st = reinterpret_cast<float4*>(&sm);
#pragma unroll
  for (int half = 0; half < C::WM; ++half) {
    __syncthreads();
    if (wm == half) stage_half<C>(st, acc, wn, lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (BM / C::WM) * (C::BN / 8) / NT; ++i) {
      const int id = threadIdx.x + NT * i;
      const int r = id / (C::BN / 8), c8 = id % (C::BN / 8);
      const float4 lo = st[r * P + ((2 * c8) ^ (r & 15))];
      const float4 hi = st[r * P + ((2 * c8 + 1) ^ (r & 15))];
      const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      body(half * (BM / C::WM) + r, c8 * 8, v);
    }
  }
}

// The plain bf16 store epilogue: the accumulators are rounded to bf16 in registers (the
// same single rounding a bf16 store of the fp32 value makes) and the whole 256 x BN tile is
// staged at once (256 x 512 B = 128 KB, all four stages), one pass through LDS instead of
// two halves of fp32. A staged row is BN/8 chunks of 8 bf16; chunk c of row r sits in slot
// c ^ (r & 15), and its two 8-byte halves trade places in rows with bit 4 set. A lane writes
// 8 bytes (4 columns of one row, 32 consecutive rows per instruction), so every 32 lanes
// cover the 64 banks once; a row read (16 bytes per lane, 16 lanes a row) spreads over all
// banks too. BODY(row, col, v) receives 8 consecutive bf16 columns of one tile row.
template <class C, class Body>
__device__ __forceinline__ void epilogue_staged_bf16(StageBufs<C>& sm, const acc_t<C>& acc, int wm, int wn,
                                                     int lane, Body body) {
  constexpr int P = C::BN / 8, NT = C::NTHR;
  static_assert(BM * C::BN * 2 <= (int)sizeof(StageBufs<C>), "the bf16 tile fits the stage buffers");
  uint2* st8 = reinterpret_cast<uint2*>(&sm);
  const uint4* st16 = reinterpret_cast<const uint4*>(&sm);
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm * (BM / C::WM) + mb * 32 + (lane & 31);
        const int col = wn * 32 * C::NB + nb * 32 + 8 * q + 4 * (lane >> 5);
        const int h = ((col >> 2) & 1) ^ ((r >> 4) & 1);
        st8[(r * P + ((col >> 3) ^ (r & 15))) * 2 + h] =
            make_uint2(pack_bf16x2(acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1]),
                       pack_bf16x2(acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]));
      }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BM * P / NT; ++i) {
    const int id = (int)threadIdx.x + NT * i;
    const int r = id / P, c = id % P;
    uint4 v = st16[r * P + (c ^ (r & 15))];
    if ((r >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
    body(r, c * 8, v);
  }
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

// ---------------------------------------------------------------- data-gradient kernel

enum { EPI_SWIGLU = 0, EPI_STORE = 1 };

struct DgradArgs {
  const uint16_t* A;   // [rows x K] packed rows (Dlt or dH), or the matrix a_rows gathers from
  int64_t lda;
  const int32_t* a_rows;  // row c of A is A[a_rows[c]] (nullptr: row c); outside [0, a_nrows): zeros
  int64_t a_nrows;
  const float* alpha;     // nullptr, or row c of the product is scaled by alpha[hc_rows[c]] (its
                          // pair's routing weight; hc_rows then maps packed rows to pairs)
  const uint16_t* W;   // [E x N x K] weights viewed as rows n with K contiguous
  int64_t ldw, w_estride;
  int N, K;            // output columns, reduction length
  int ntn;             // ceil(N / CfgD::BN)
  const int64_t* row_off;
  int E;
  // epilogue
  const uint16_t* HC;  // SwiGLU: saved [gate | up] rows, 2F wide
  const int32_t* hc_rows;  // row of HC (and pair of alpha) for packed row c (nullptr: row c)
  int64_t hc_nrows;        // rows of HC: a mapped row outside [0, hc_nrows) reads as zeros
  uint16_t* out;       // SwiGLU: dH [rows x 2F]; STORE: [rows x N]
  int64_t ldo;
  int F;
};

// SwiGLU backward epilogue of the FC2 data gradient: the tile's dPhi (the accumulators) gives
// dH = [dPhi * up * silu'(gate), dPhi * silu(gate)] with gate, up read from the saved rows.
// Staged through LDS in two halves like epilogue_staged. The tile's HC rows (the row map,
// fetched before the K loop) and their routing weights reach every thread through LDS
// (ep_rows, ep_alpha), so the first [gate | up] loads of a half depend on no global load.
// A thread handles kIt rows per half: it loads their [gate | up] chunks in batches of 4 rows,
// each batch's loads issued before the previous batch is computed, and stores a batch's dH
// only after computing all of it, so a half costs a few overlapping memory round trips
// instead of three per row. The first batch is loaded before the half is staged. (With eight
// wavefronts the kernel then holds 256 VGPRs without spilling: two batches in flight beside
// the accumulators of the half not yet staged. Against running the first half's two batches
// one after the other and the second half as one batch of 8: FC2 data gradient 1.8% faster
// at the Qwen3 share, 1.2% at the GLM share.) Loads always read a valid address (row 0 for a
// row outside the tile or outside HC) and such a row gets a zero weight, which zeroes its dH
// (the saved rows are finite), so the compiler neither branches around the loads nor waits
// between them.
template <int B>
struct HcBatch {
  uint4 gw[B], uw[B];
};

template <class C, int B, bool AHEAD, class Pre>
__device__ __forceinline__ void swiglu_half(StageBufs<C>& sm, const acc_t<C>& acc, int wm, int wn, int lane,
                                            const DgradArgs& g, const int32_t* ep_rows, const float* ep_alpha,
                                            int64_t row0, int rows_valid, int n0, int n_valid, int half, Pre pre) {
  constexpr int BN = C::BN, NTHR = C::NTHR, P = BN / 4;
  constexpr int kIt = (BM / C::WM) * (BN / 8) / NTHR;  // rows per thread per half
  constexpr int kRowStep = NTHR / (BN / 8);
  constexpr int kNb = kIt / B;
  static_assert(kNb * B == kIt, "whole batches");
  const int tr0 = threadIdx.x / (BN / 8), tc = (threadIdx.x % (BN / 8)) * 8;
  const int64_t ld = 2 * (int64_t)g.F;
  const int F = g.F;
  const bool col_ok = tc < n_valid;
  const uint16_t* __restrict__ hc = g.HC;
  uint16_t* __restrict__ dh = g.out;
  float4* st = reinterpret_cast<float4*>(&sm);
  auto issue = [&](HcBatch<B>& bt, int i0) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int32_t hr = ep_rows[half * (BM / C::WM) + tr0 + kRowStep * (i0 + b)];
      const int64_t hb = hr >= 0 && col_ok ? (int64_t)hr * ld + n0 + tc : 0;
      bt.gw[b] = *(const uint4*)(hc + hb);
      bt.uw[b] = *(const uint4*)(hc + hb + F);
    }
  };
  auto finish = [&](HcBatch<B>& bt, int i0) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int r = tr0 + kRowStep * (i0 + b), c8 = tc / 8;
      const float4 lo = st[r * P + ((2 * c8) ^ (r & 15))];
      const float4 hi = st[r * P + ((2 * c8 + 1) ^ (r & 15))];
      // the row's routing weight; 0 for a row outside the tile or HC, whose [gate | up]
      // words are row 0's, so its dH is zero
      const float av = col_ok ? ep_alpha[half * (BM / C::WM) + r] : 0.0f;
      const float dphi[8] = {av * lo.x, av * lo.y, av * lo.z, av * lo.w, av * hi.x, av * hi.y, av * hi.z, av * hi.w};
      const uint32_t gg[4] = {bt.gw[b].x, bt.gw[b].y, bt.gw[b].z, bt.gw[b].w};
      const uint32_t uu[4] = {bt.uw[b].x, bt.uw[b].y, bt.uw[b].z, bt.uw[b].w};
      float dg[8], du[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float gate = (c & 1) ? bf16_hi(gg[c >> 1]) : bf16_lo(gg[c >> 1]);
        const float up = (c & 1) ? bf16_hi(uu[c >> 1]) : bf16_lo(uu[c >> 1]);
        // sigmoid from the hardware base-2 exponential and reciprocal (about 1 ulp each; the
        // result is rounded to bf16): 1 / (1 + 2^(-gate log2 e))
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gate * -1.44269504088896341f));
        // silu(gate) = gate sg; silu'(gate) = sg (1 + gate (1 - sg)) = sg + silu(gate) (1 - sg)
        const float sl = gate * sg;
        dg[c] = dphi[c] * up * __builtin_fmaf(sl, 1.0f - sg, sg);
        du[c] = dphi[c] * sl;
      }
      bt.gw[b] = pack_bf16x8(dg);
      bt.uw[b] = pack_bf16x8(du);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int tr = half * (BM / C::WM) + tr0 + kRowStep * (i0 + b);
      if (tr < rows_valid && col_ok) {
        const int64_t rowb = (row0 + tr) * ld + n0 + tc;
        *(uint4*)(dh + rowb) = bt.gw[b];
        *(uint4*)(dh + rowb + F) = bt.uw[b];
      }
    }
  };
  HcBatch<B> bt[kNb > 1 ? 2 : 1];
  issue(bt[0], 0);
  pre();
  __syncthreads();
  if (wm == half) stage_half<C>(st, acc, wn, lane);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kNb; ++i) {
    if (AHEAD && i + 1 < kNb) issue(bt[(i + 1) & 1], (i + 1) * B);
    finish(bt[i & 1], i * B);
    if (!AHEAD && i + 1 < kNb) issue(bt[(i + 1) & 1], (i + 1) * B);
  }
}

// my_row: for threads below BM, the HC row of tile row threadIdx.x (-1: none), loaded before
// the K loop. Its routing weight is loaded here, beside the first [gate | up] loads, and
// written to LDS before the first half is staged.
template <class C>
__device__ __forceinline__ void epilogue_swiglu(StageBufs<C>& sm, const acc_t<C>& acc, int wm, int wn, int lane,
                                                const DgradArgs& g, int32_t* ep_rows, float* ep_alpha,
                                                int32_t my_row, int64_t row0, int rows_valid, int n0,
                                                int n_valid) {
  static_assert(C::WM == 2, "two halves");
  const int t = threadIdx.x;
  if (t < BM) ep_rows[t] = my_row;
  float my_alpha = 0.0f;
  if (t < BM && my_row >= 0) my_alpha = g.alpha != nullptr ? g.alpha[my_row] : 1.0f;
  __syncthreads();
  auto pre0 = [&] {
    if (t < BM) ep_alpha[t] = my_alpha;
  };
  auto pre1 = [] {};
  swiglu_half<C, 4, true>(sm, acc, wm, wn, lane, g, ep_rows, ep_alpha, row0, rows_valid, n0, n_valid, 0, pre0);
  swiglu_half<C, 4, true>(sm, acc, wm, wn, lane, g, ep_rows, ep_alpha, row0, rows_valid, n0, n_valid, 1, pre1);
}

// The kernel's one LDS object: the stage buffers (both forms), then for EPI_SWIGLU the
// epilogue's row map.
template <class C, int EPI>
struct DgradShared {
  union {
    StageBufs<C> st;  // the epilogue's staging
    StageBufs64 k64;  // the K loop
  };
};
template <class C>
struct DgradShared<C, EPI_SWIGLU> {
  union {
    StageBufs<C> st;
    StageBufs64 k64;
  };
  int32_t ep_rows[BM];  // SwiGLU epilogue: HC row of each tile row (-1: none)
  float ep_alpha[BM];   // and its routing weight
};

// One output tile per block.
template <int EPI>
__global__ LRMOE_GEMM_ATTR(CfgD) void dgrad_kernel(DgradArgs g) {
  using C = CfgD;
  // one LDS object: the stage buffers, then the SwiGLU epilogue's row map (with a second
  // __shared__ variable the compiler attaches alias scopes to LDS accesses and then waits
  // for every direct load before each fragment read)
  __shared__ DgradShared<C, EPI> lds_all;
  StageBufs<C>& lds = lds_all.st;
  const int b = xcd_remap(blockIdx.x, gridDim.x);
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
  const int n0 = nt * C::BN;
  const int n_valid = min(C::BN, g.N - n0);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  // SwiGLU epilogue: thread t < BM fetches tile row t's HC row now, so that the value is in a
  // register by the end of the K loop
  int32_t my_row = -1;
  if (EPI == EPI_SWIGLU && (int)threadIdx.x < rows_valid) {
    const int64_t j = g.hc_rows != nullptr ? (int64_t)g.hc_rows[row0 + threadIdx.x] : row0 + threadIdx.x;
    my_row = j >= 0 && j < g.hc_nrows ? (int32_t)j : -1;
  }
  acc_t<C> acc;
  zero_acc<C>(acc);
  auto init = [&](auto& la, auto& lb) {
    if (g.a_rows != nullptr) la.init_rows(g.A, g.lda, rows_valid, g.a_rows + row0, g.a_nrows);
    else la.init(g.A + row0 * g.lda, g.lda, rows_valid);
    lb.init(g.W + (int64_t)e * g.w_estride + (int64_t)n0 * g.ldw, g.ldw, n_valid);
  };
  // The 64-K loop: whole-line requests. Against the 32-K loop, alternating builds: FC1 data
  // gradient 3-4% faster on the Qwen3 and GLM shares, FC2 data gradient 0.4-1.3%.
  DmaK64<C::NWAVE, BM> la;
  DmaK64<C::NWAVE, C::BN> lb;
  init(la, lb);
  gemm_mainloop_k64<C>(lds_all.k64, la, lb, g.K, acc, wm, wn, lane);

  if constexpr (EPI == EPI_SWIGLU) {
    epilogue_swiglu<C>(lds, acc, wm, wn, lane, g, lds_all.ep_rows, lds_all.ep_alpha, my_row, row0, rows_valid, n0,
                       n_valid);
  } else if (g.alpha == nullptr) {  // uniform
    uint16_t* __restrict__ out = g.out;
    epilogue_staged_bf16<C>(lds, acc, wm, wn, lane, [&](int tr, int tc, const uint4& v) {
      if (tr < rows_valid && tc < n_valid) *(uint4*)(out + (row0 + tr) * g.ldo + n0 + tc) = v;
    });
  } else {  // each row scaled by its pair's routing weight in fp32 before the rounding
    uint16_t* __restrict__ out = g.out;
    epilogue_staged<C>(lds, acc, wm, wn, lane, [&](int tr, int tc, const float (&v)[8]) {
      if (tr < rows_valid && tc < n_valid) {
        const int64_t j = g.hc_rows[row0 + tr];
        const float av = j >= 0 && j < g.hc_nrows ? g.alpha[j] : 0.0f;
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = av * v[i];
        *(uint4*)(out + (row0 + tr) * g.ldo + n0 + tc) = pack_bf16x8(w);
      }
    });
  }
}

// ---------------------------------------------------------------- forward with context save
//
// The expert forward that produces the backward's saved context (Algorithm 1's
// FullForwardAndSaveContext; section 3.1 keeps every routed pair in the forward). Pair j of
// expert e, over all N pairs in expert-major order:
//   FC1  h_j = x_{tok[j]} W1[e]          X rows gathered through tok, W1[e] read [D x 2F]
//   SwiGLU phi_j = silu(gate_j) * up_j   fused in the FC1 epilogue; H and Phi saved in bf16
//   FC2  y_j = alpha_j * phi_j W2[e]     the stored phi, W2[e] read [F x D]; Y rows in bf16
// The layer output is the token sum of the Y rows (the scatter step).

struct FwdArgs {
  const uint16_t* X;    // [T x D] token rows
  int64_t T;
  const int32_t* tok;   // [N] token of each pair
  const float* alpha;   // [N] routing weights
  const uint16_t* W1;   // [E x D x 2F]
  const uint16_t* W2;   // [E x F x D]
  uint16_t* H;          // [N x 2F] out
  uint16_t* Phi;        // [N x F] out (FC1 launch) / in (FC2 launch)
  uint16_t* Y;          // [N x D] out
  const int64_t* row_off;
  int E, D, F;
  int ntn;              // N tiles per M tile: ceil(F / 128) (FC1), ceil(D / 256) (FC2)
};

// Expert, first row and rows of M tile `local / ntn` (uniform per block); false past the end.
__device__ __forceinline__ bool fwd_tile(const FwdArgs& g, int b, int& e, int64_t& row0, int& rows_valid, int& nt) {
  int local = b;
  for (e = 0; e < g.E; ++e) {
    const int64_t r0 = g.row_off[e], m = g.row_off[e + 1] - r0;
    const int cnt = (int)((m + BM - 1) / BM) * g.ntn;
    if (local < cnt) {
      const int mt = local / g.ntn;
      nt = local % g.ntn;
      row0 = r0 + (int64_t)mt * BM;
      rows_valid = (int)min<int64_t>(BM, m - (int64_t)mt * BM);
      return true;
    }
    local -= cnt;
  }
  return false;
}

// FC1 tile: 256 pair rows x [128 gate | 128 up] columns j0 = 128 nt; the SwiGLU forward in the
// epilogue, staged through LDS like epilogue_staged. A thread takes 8 gate columns of a row
// with the matching 8 up columns and writes both to H and phi = silu(gate) * up (from the
// fp32 sums, rounded once) to Phi.
__global__ LRMOE_GEMM_ATTR(CfgW) void fwd_fc1_kernel(FwdArgs g) {
  using C = CfgW;
  __shared__ StageBufs<C> lds;
  int e, rows_valid, nt;
  int64_t row0;
  if (!fwd_tile(g, xcd_remap(blockIdx.x, gridDim.x), e, row0, rows_valid, nt)) return;  // uniform per block
  const int j0 = nt * 128, F = g.F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  acc_t<C> acc;
  zero_acc<C>(acc);
  DmaK<C::NWAVE, BM> la;
  la.init_rows(g.X, g.D, rows_valid, g.tok + row0, g.T);
  DmaT<C::NL> lb;
  lb.init_paired(g.W1 + (int64_t)e * g.D * 2 * F, 2 * F, j0, F);
  gemm_mainloop<C, false, true>(lds, la, lb, g.D, 0, (uint32_t)(2 * F * 2), acc, wm, wn, lane);

  constexpr int P = C::BN / 4;  // float4 per staged row
  float4* st = reinterpret_cast<float4*>(&lds);
  const int64_t ldh = 2 * (int64_t)F;
#pragma unroll
  for (int half = 0; half < C::WM; ++half) {
    __syncthreads();
    if (wm == half) stage_half<C>(st, acc, wn, lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (BM / C::WM) * 16 / C::NTHR; ++i) {
      const int id = threadIdx.x + C::NTHR * i;
      const int r = id / 16, c8 = id % 16;
      const int tr = half * (BM / C::WM) + r, f = j0 + c8 * 8;
      if (tr < rows_valid && f < F) {
        const float4 g0 = st[r * P + ((2 * c8) ^ (r & 15))], g1 = st[r * P + ((2 * c8 + 1) ^ (r & 15))];
        const float4 u0 = st[r * P + ((32 + 2 * c8) ^ (r & 15))], u1 = st[r * P + ((32 + 2 * c8 + 1) ^ (r & 15))];
        const float gt[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float ut[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float ph[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          // silu from the hardware base-2 exponential and reciprocal: x / (1 + 2^(-x log2 e))
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gt[k] * -1.44269504088896341f));
          ph[k] = gt[k] * sg * ut[k];
        }
        const int64_t row = row0 + tr;
        *(uint4*)(g.H + row * ldh + f) = pack_bf16x8(gt);
        *(uint4*)(g.H + row * ldh + F + f) = pack_bf16x8(ut);
        *(uint4*)(g.Phi + row * F + f) = pack_bf16x8(ph);
      }
    }
  }
}

// FC2 tile: 256 pair rows x 256 output columns n0 = 256 nt; rows scaled by their routing
// weight in the epilogue.
__global__ LRMOE_GEMM_ATTR(CfgW) void fwd_fc2_kernel(FwdArgs g) {
  using C = CfgW;
  __shared__ StageBufs<C> lds;
  int e, rows_valid, nt;
  int64_t row0;
  if (!fwd_tile(g, xcd_remap(blockIdx.x, gridDim.x), e, row0, rows_valid, nt)) return;  // uniform per block
  const int n0 = nt * C::BN, n_valid = min(C::BN, g.D - n0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  acc_t<C> acc;
  zero_acc<C>(acc);
  DmaK<C::NWAVE, BM> la;
  la.init(g.Phi + row0 * g.F, g.F, rows_valid);
  DmaT<C::NL> lb;
  lb.init(g.W2 + (int64_t)e * g.F * g.D + n0, g.D, n_valid);
  gemm_mainloop<C, false, true>(lds, la, lb, g.F, 0, (uint32_t)(g.D * 2), acc, wm, wn, lane);
  uint16_t* __restrict__ y = g.Y;
  const float* __restrict__ alpha = g.alpha;
  const int D = g.D;
  epilogue_staged<C>(lds, acc, wm, wn, lane, [&](int tr, int tc, const float (&v)[8]) {
    if (tr < rows_valid && tc < n_valid) {
      const float a = alpha[row0 + tr];
      const float w[8] = {a * v[0], a * v[1], a * v[2], a * v[3], a * v[4], a * v[5], a * v[6], a * v[7]};
      *(uint4*)(y + (row0 + tr) * D + n0 + tc) = pack_bf16x8(w);
    }
  });
}

// ---------------------------------------------------------------- weight-gradient kernels

struct WgradType {
  const uint16_t* A;  // [rows x M] (M contiguous), or the matrix that a_rows gathers from
  int64_t lda;
  const int32_t* a_rows;  // packed row c is row a_rows[c] of A (nullptr: row c)
  int64_t a_nrows;        // rows of A when gathered
  const uint16_t* B;  // [rows x N] (N contiguous), or the matrix that b_rows gathers from
  int64_t ldb;
  float* out;         // [E x M x N]
  int M, N, ntm, ntn, tiles;
  const int32_t* b_rows;  // packed row c is row b_rows[c] of B (nullptr: row c)
  int64_t b_nrows;        // rows of B when gathered
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
  int64_t kc_max;       // longest chunk (packed rows), chosen by the host
  // Items (planned order) of XCD x: [xlo[x], xlo[x+1]). The ranges are contiguous, so the
  // tiles sharing operand panels stay in one L2, and cut so every XCD gets the same number
  // of K steps: items are sorted by decreasing length, so equal item counts would hand the
  // first XCD several times the work of the last.
  int xlo[9];
};

__host__ __device__ inline void expert_split(int64_t m, int64_t kc_max, int& s, int& kc) {
  if (m <= 0) {
    s = 1;
    kc = 0;
    return;
  }
  const int64_t sc = (m + kc_max - 1) / kc_max;
  const int64_t per = (m + sc - 1) / sc;
  s = (int)sc;
  kc = (int)((per + BK - 1) / BK * BK);
}

// Block-wide inclusive prefix sum in thread order over kAuxThr threads; the block total in
// tot. Every thread of the block must call it.
template <class T>
__device__ __forceinline__ T plan_scan(T v, T& tot, T* sh) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  T inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  T pre = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < kAuxThr / kWave; ++w) {
    if (w < wave) pre += sh[w];
    tot += sh[w];
  }
  __syncthreads();
  return pre + inc;
}

// One block: order experts by decreasing chunk length (ties: lower id) and lay out items.
__global__ __launch_bounds__(kAuxThr) void wgrad_plan_kernel(WgradArgs g) {
  const int E = g.E;
  const int tiles = g.t[0].tiles + (g.ntypes > 1 ? g.t[1].tiles : 0);
  for (int e = threadIdx.x; e < E; e += kAuxThr) {
    int s, kc;
    expert_split(g.row_off[e + 1] - g.row_off[e], g.kc_max, s, kc);
    g.plan_s[e] = s;
    g.plan_kc[e] = kc;
  }
  __syncthreads();
  // rank of each expert in the planned order: the chunk lengths are compared from LDS,
  // kAuxThr experts at a time
  __shared__ int kc_sh[kAuxThr];
  for (int e0 = 0; e0 < E; e0 += kAuxThr) {  // uniform trip count
    const int e = e0 + (int)threadIdx.x;
    const int kc = e < E ? g.plan_kc[e] : 0;
    int rank = 0;
    for (int f0 = 0; f0 < E; f0 += kAuxThr) {
      __syncthreads();
      kc_sh[threadIdx.x] = f0 + (int)threadIdx.x < E ? g.plan_kc[f0 + threadIdx.x] : 0;
      __syncthreads();
      const int nf = min(kAuxThr, E - f0);
      for (int j = 0; j < nf; ++j) {
        const int kf = kc_sh[j], f = f0 + j;
        rank += (kf > kc || (kf == kc && f < e)) ? 1 : 0;
      }
    }
    if (e < E) g.plan_e[rank] = e;
  }
  __syncthreads();
  // items before each planned expert, and each split expert's first partial tile (expert id
  // order): exclusive prefix sums, kAuxThr experts at a time
  __shared__ int sh_i[kAuxThr / kWave];
  __shared__ int64_t sh_p[kAuxThr / kWave];
  int items_before = 0;
  int64_t parts_before = 0;
  for (int r0 = 0; r0 < E; r0 += kAuxThr) {  // uniform trip count
    const int r = r0 + (int)threadIdx.x;
    const int items = r < E ? g.plan_s[g.plan_e[r]] * tiles : 0;
    const int sr = r < E ? g.plan_s[r] : 1;
    const int64_t parts = sr > 1 ? (int64_t)sr * tiles : 0;
    int ti;
    int64_t tp;
    const int ii = plan_scan<int>(items, ti, sh_i);
    const int64_t ip = plan_scan<int64_t>(parts, tp, sh_p);
    if (r < E) {
      g.plan_prefix[r] = items_before + ii - items;
      g.plan_pbase[r] = parts_before + ip - parts;
    }
    items_before += ti;
    parts_before += tp;
  }
  if (threadIdx.x == 0) g.plan_prefix[E] = items_before;
}

// G0, G1: the A operand of weight-gradient type 0 (FC2: Phi) / type 1 (FC1: X) is gathered
// through its row map; GB0: the B operand of type 0 (the gradient rows) is (compile-time
// choices, so no loader carries another's code).
template <bool G0, bool G1, bool GB0>
__global__ LRMOE_GEMM_ATTR(CfgW) void wgrad_kernel(WgradArgs g) {
  static_assert(!(G0 && GB0), "type 0 gathers at most one operand");
  using C = CfgW;
  __shared__ StageBufs<C> lds;
  // hardware sends block i to XCD i % 8; the grid holds 8 x (largest range) blocks
  const int x = blockIdx.x & 7;
  const int b = g.xlo[x] + (int)(blockIdx.x >> 3);
  if (b >= g.xlo[x + 1]) return;  // uniform per block
  int lo = 0, hi = g.E;  // planned expert r with prefix[r] <= b < prefix[r+1]
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

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  acc_t<C> acc;
  zero_acc<C>(acc);
  if (GB0 && ty == 0) {  // packed A, gathered B
    DmaT<C::NL> la;
    DmaTG<C::NL> lb;
    la.init(T.A + (r0 + k_begin) * T.lda + m0, T.lda, m_valid);
    lb.init(T.B + n0, T.ldb, n_valid, T.b_rows + r0 + k_begin, klen, T.b_nrows);
    gemm_mainloop<C, true, true>(lds, la, lb, klen, (uint32_t)(T.lda * 2), 0, acc, wm, wn, lane);
  } else if ((G0 || G1) && (ty == 0 ? G0 : G1)) {  // gathered A, packed B
    DmaTG<C::NL> la;
    DmaT<C::NL> lb;
    la.init(T.A + m0, T.lda, m_valid, T.a_rows + r0 + k_begin, klen, T.a_nrows);
    lb.init(T.B + (r0 + k_begin) * T.ldb + n0, T.ldb, n_valid);
    gemm_mainloop<C, true, true>(lds, la, lb, klen, 0, (uint32_t)(T.ldb * 2), acc, wm, wn, lane);
  } else {
    DmaT<C::NL> la, lb;
    la.init(T.A + (r0 + k_begin) * T.lda + m0, T.lda, m_valid);
    lb.init(T.B + (r0 + k_begin) * T.ldb + n0, T.ldb, n_valid);
    gemm_mainloop<C, true, true>(lds, la, lb, klen, (uint32_t)(T.lda * 2), (uint32_t)(T.ldb * 2), acc, wm, wn, lane);
  }

  if (s > 1) {
    float* __restrict__ p = g.partials + (g.plan_pbase[e] + (int64_t)chunk * tiles + rem) * (int64_t)(BM * BN);
    epilogue_staged<C>(lds, acc, wm, wn, lane, [&](int tr, int tc, const float (&v)[8]) {
      float4* q4 = (float4*)(p + tr * BN + tc);
      q4[0] = make_float4(v[0], v[1], v[2], v[3]);
      q4[1] = make_float4(v[4], v[5], v[6], v[7]);
    });
  } else {
    float* __restrict__ o = T.out + (int64_t)e * T.M * T.N;
    const bool accum = g.accumulate != 0;
    epilogue_staged<C>(lds, acc, wm, wn, lane, [&](int tr, int tc, const float (&v)[8]) {
      if (tr < m_valid && tc < n_valid) {
        float4* q4 = (float4*)(o + (int64_t)(m0 + tr) * T.N + n0 + tc);
        float4 a = make_float4(v[0], v[1], v[2], v[3]), b = make_float4(v[4], v[5], v[6], v[7]);
        if (accum) {
          const float4 oa = q4[0], ob = q4[1];
          a.x += oa.x; a.y += oa.y; a.z += oa.z; a.w += oa.w;
          b.x += ob.x; b.y += ob.y; b.z += ob.z; b.w += ob.w;
        }
        q4[0] = a;
        q4[1] = b;
      }
    });
  }
}

// Sums the chunk partials of every split tile in chunk order into the output. Each tile is
// shared by kRedParts blocks of BM / kRedParts rows, so enough blocks are in flight to
// cover the partials' read latency; a thread keeps its four float4 loads of a chunk in
// flight together.
constexpr int kRedParts = 8;
constexpr int kRedPer = BM / kRedParts * (BN / 4) / kAuxThr;  // float4 per thread (4)

__global__ __launch_bounds__(kAuxThr) void wgrad_reduce_kernel(WgradArgs g) {
  const int tiles = g.t[0].tiles + (g.ntypes > 1 ? g.t[1].tiles : 0);
  const int part = blockIdx.x % kRedParts;
  int b = blockIdx.x / kRedParts, e = 0;
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
  int r[kRedPer], c[kRedPer];
  bool ok[kRedPer];
  float4 sum[kRedPer];
#pragma unroll
  for (int u = 0; u < kRedPer; ++u) {
    const int idx = part * (BM / kRedParts) * (BN / 4) + threadIdx.x + u * kAuxThr;
    r[u] = idx / (BN / 4);
    c[u] = (idx % (BN / 4)) * 4;
    ok[u] = r[u] < m_valid && c[u] < n_valid;
    sum[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int ch = 0; ch < s; ++ch) {
    float4 v[kRedPer];
#pragma unroll
    for (int u = 0; u < kRedPer; ++u)
      v[u] = ok[u] ? *(const float4*)(p0 + ch * pstride + r[u] * BN + c[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kRedPer; ++u) {
      sum[u].x += v[u].x;
      sum[u].y += v[u].y;
      sum[u].z += v[u].z;
      sum[u].w += v[u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < kRedPer; ++u) {
    if (!ok[u]) continue;
    float4* q = (float4*)(o + (int64_t)(m0 + r[u]) * T.N + n0 + c[u]);
    float4 t = sum[u];
    if (g.accumulate) {
      const float4 old = *q;
      t.x += old.x;
      t.y += old.y;
      t.z += old.z;
      t.w += old.w;
    }
    *q = t;
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

// out[r][n] = a(r) sum_k A[ar(r)][k] * W[e(r)][n][k]; SwiGLU epilogue or plain store. ar(r) =
// a_rows[r] (rows outside [0, a_nrows) read as zeros) or r; a(r) = alpha[hc_rows[r]] or 1.
template <int EPI>
__global__ __launch_bounds__(kAuxThr) void f32_dgrad_kernel(const float* __restrict__ A, int64_t lda,
                                                         const int32_t* __restrict__ a_rows, int64_t a_nrows,
                                                         const float* __restrict__ alpha,
                                                         const float* __restrict__ W, int64_t ldw,
                                                         int64_t w_estride, int N, int K,
                                                         const int64_t* __restrict__ row_off, int E,
                                                         const float* __restrict__ HC,
                                                         const int32_t* __restrict__ hc_rows, int64_t hc_nrows,
                                                         float* __restrict__ out, int64_t ldo, int F) {
  const int64_t r = blockIdx.x;
  const int n = blockIdx.y * kAuxThr + threadIdx.x;
  if (n >= N) return;
  const int e = find_expert(row_off, E, r);
  const int64_t ar = a_rows != nullptr ? (int64_t)a_rows[r] : r;
  const bool a_ok = a_rows == nullptr || (ar >= 0 && ar < a_nrows);
  const float* a = A + (a_ok ? ar : 0) * lda;
  const float* w = W + (int64_t)e * w_estride + (int64_t)n * ldw;
  float acc = 0.0f;
  if (a_ok)
    for (int k = 0; k < K; ++k) acc = fmaf(a[k], w[k], acc);
  const int64_t hr = hc_rows != nullptr ? (int64_t)hc_rows[r] : r;
  const bool ok = hr >= 0 && hr < hc_nrows;  // rows outside HC read as zeros
  if (alpha != nullptr) acc *= ok ? alpha[hr] : 0.0f;
  if (EPI == EPI_SWIGLU) {
    const float gate = ok ? HC[hr * 2 * F + n] : 0.0f, up = ok ? HC[hr * 2 * F + F + n] : 0.0f;
    const float s = 1.0f / (1.0f + expf(-gate));
    out[r * 2 * F + n] = acc * up * (s * (1.0f + gate * (1.0f - s)));
    out[r * 2 * F + F + n] = acc * (gate * s);
  } else {
    out[r * ldo + n] = acc;
  }
}

// out[e][i][j] (+)= sum over rows r of expert e of A[ar(r)][i] * B[br(r)][j], with ar(r) =
// a_rows[r] (rows outside [0, a_nrows) read as zeros) or r when a_rows is nullptr, and br
// likewise from b_rows
__global__ __launch_bounds__(kAuxThr) void f32_wgrad_kernel(const float* __restrict__ A, int64_t lda,
                                                         const int32_t* __restrict__ a_rows, int64_t a_nrows,
                                                         const float* __restrict__ B, int64_t ldb,
                                                         const int32_t* __restrict__ b_rows, int64_t b_nrows,
                                                         int M, int N,
                                                         const int64_t* __restrict__ row_off,
                                                         float* __restrict__ out, int accumulate) {
  const int e = blockIdx.z, i = blockIdx.y;
  const int j = blockIdx.x * kAuxThr + threadIdx.x;
  if (j >= N) return;
  float acc = 0.0f;
  for (int64_t r = row_off[e]; r < row_off[e + 1]; ++r) {
    const int64_t ar = a_rows != nullptr ? (int64_t)a_rows[r] : r;
    const float a = (a_rows == nullptr || (ar >= 0 && ar < a_nrows)) ? A[ar * lda + i] : 0.0f;
    const int64_t br = b_rows != nullptr ? (int64_t)b_rows[r] : r;
    const float b = (b_rows == nullptr || (br >= 0 && br < b_nrows)) ? B[br * ldb + j] : 0.0f;
    acc = fmaf(a, b, acc);
  }
  float* q = out + ((int64_t)e * M + i) * N + j;
  *q = accumulate ? *q + acc : acc;
}

// ---------------------------------------------------------------- host side

struct WgradLayout {
  size_t plan_bytes, partial_bytes;
  int64_t npartials, nitems, nreduce;
};

int wgrad_tiles(int M, int N) { return (int)(ceil_div(M, BM) * ceil_div(N, BN)); }

WgradLayout wgrad_layout(const lrmoe_problem* p, const int64_t* row_off_h, int64_t kc_max) {
  const int tiles = wgrad_tiles(p->F, p->D) + (p->swiglu ? wgrad_tiles(p->D, 2 * p->F) : 0);
  WgradLayout L{};
  for (int e = 0; e < p->E; ++e) {
    const int64_t m = row_off_h[e + 1] - row_off_h[e];
    const int64_t s = m <= 0 ? 1 : ceil_div(m, kc_max);
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

// The weight-gradient schedule of one problem: the chunk length and the items' split into 8
// contiguous ranges, one per XCD (hardware sends block i to XCD i % 8).
struct WgradSchedule {
  int64_t kc_max;
  int xlo[9];
  int64_t per_xcd;  // items of the largest range
};

// Items in the order the plan kernel gives them (experts by decreasing chunk length, ties by
// id; chunk-major within an expert), cut into 8 contiguous ranges. An item costs its K steps
// plus 8 for its prologue and epilogue. The cut minimises the largest range's finishing time
// when its 32 CUs take items in order as they free up: a bisection on that time, each probe
// filling the ranges greedily. Returns that time. Any monotone split covers every item
// exactly once, so the split only affects balance, never results.
int64_t wgrad_xcd_ranges(const lrmoe_problem* p, const int64_t* row_off_h, int64_t kc_max, int (&xlo)[9]) {
  constexpr int kXcd = 8, kCuPerXcd = 32;
  const int E = p->E;
  const int tiles = wgrad_tiles(p->F, p->D) + (p->swiglu ? wgrad_tiles(p->D, 2 * p->F) : 0);
  std::vector<int> order(E), S(E), KC(E);
  for (int e = 0; e < E; ++e) {
    order[e] = e;
    expert_split(row_off_h[e + 1] - row_off_h[e], kc_max, S[e], KC[e]);
  }
  std::sort(order.begin(), order.end(), [&](int a, int b) { return KC[a] != KC[b] ? KC[a] > KC[b] : a < b; });
  std::vector<int64_t> cost;  // per item, planned order
  for (int e : order) {
    const int64_t m = row_off_h[e + 1] - row_off_h[e];
    for (int c = 0; c < S[e]; ++c) {
      const int64_t klen = std::max<int64_t>(0, std::min<int64_t>(KC[e], m - (int64_t)c * KC[e]));
      cost.insert(cost.end(), tiles, ceil_div(klen, BK) + 8);
    }
  }
  const int64_t n = (int64_t)cost.size();
  int64_t total = 0, longest = 0;
  for (int64_t c : cost) {
    total += c;
    longest = std::max(longest, c);
  }
  // fills the ranges so that no CU finishes after T; false if items are left over
  auto fill = [&](int64_t T, int (&lo)[9]) {
    int64_t i = 0;
    lo[0] = 0;
    for (int x = 0; x < kXcd; ++x) {
      std::vector<int64_t> cu(kCuPerXcd, 0);  // min-heap of CU finishing times
      std::make_heap(cu.begin(), cu.end(), std::greater<int64_t>());
      while (i < n && cu.front() + cost[i] <= T) {
        std::pop_heap(cu.begin(), cu.end(), std::greater<int64_t>());
        cu.back() += cost[i++];
        std::push_heap(cu.begin(), cu.end(), std::greater<int64_t>());
      }
      lo[x + 1] = (int)i;
    }
    return i == n;
  };
  // bracket the answer by doubling from its lower bound (it is rarely far above it), then bisect
  int64_t lo_t = std::max(longest, ceil_div(total, (int64_t)kXcd * kCuPerXcd)), hi_t = lo_t;
  for (int tmp[9]; !fill(hi_t, tmp);) {
    lo_t = hi_t + 1;
    hi_t = std::min(total, 2 * hi_t);
  }
  while (lo_t < hi_t) {
    const int64_t mid = lo_t + (hi_t - lo_t) / 2;
    int tmp[9];
    if (fill(mid, tmp)) hi_t = mid;
    else lo_t = mid + 1;
  }
  fill(lo_t, xlo);
  return lo_t;
}

// Chooses the chunk length among kKcCandidates: contiguous XCD ranges balance well only when
// the items are small against a range, so one dominant expert (most of the retained rows)
// gets shorter chunks, while shorter chunks cost partial tiles that the split-K reduction
// streams. Modelled time, in K steps per CU: the ranges' finishing time plus 1/16 step per
// partial tile (a 256 x 256 fp32 tile written once and read once, over the whole chip).
WgradSchedule wgrad_schedule_compute(const lrmoe_problem* p, const int64_t* row_off_h) {
  WgradSchedule best{};
  int64_t best_cost = -1;
  for (int64_t kc : kKcCandidates) {
    WgradSchedule w{};
    w.kc_max = kc;
    const int64_t t = wgrad_xcd_ranges(p, row_off_h, kc, w.xlo);
    const int64_t cost = t + wgrad_layout(p, row_off_h, kc).npartials / 16;
    if (best_cost < 0 || cost < best_cost) {
      best = w;
      best_cost = cost;
    }
  }
  for (int x = 0; x < 8; ++x) best.per_xcd = std::max<int64_t>(best.per_xcd, best.xlo[x + 1] - best.xlo[x]);
  return best;
}

// The schedule costs about a millisecond of host time for a 128-expert layer, and a training
// loop asks for the same routing's schedule several times (workspace size, then the launch),
// so the last few are kept, keyed by everything the schedule reads.
WgradSchedule wgrad_schedule(const lrmoe_problem* p, const int64_t* row_off_h) {
  constexpr int kKeep = 8;
  struct Entry {
    std::vector<int64_t> key;
    WgradSchedule sched;
  };
  static std::mutex mu;
  static Entry memo[kKeep];
  static int next = 0;
  std::vector<int64_t> key = {p->E, p->D, p->F, p->swiglu};
  key.reserve(4 + (size_t)p->E);
  for (int e = 0; e < p->E; ++e) key.push_back(row_off_h[e + 1] - row_off_h[e]);
  {
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry& m : memo)
      if (m.key == key) return m.sched;
  }
  const WgradSchedule w = wgrad_schedule_compute(p, row_off_h);
  std::lock_guard<std::mutex> lk(mu);
  memo[next] = Entry{std::move(key), w};
  next = (next + 1) % kKeep;
  return w;
}

}  // namespace

lrmoe_status launch_expert_forward(const lrmoe_problem* p, const int64_t* seg_off_d, const void* X,
                                   const int32_t* tok, const float* alpha, const void* W1, const void* W2, void* H,
                                   void* Phi, void* Y, hipStream_t s) {
  int64_t mtiles = 0;
  for (int e = 0; e < p->E; ++e) mtiles += ceil_div(p->seg_off[e + 1] - p->seg_off[e], BM);
  if (mtiles == 0) return LRMOE_OK;
  FwdArgs g{};
  g.X = (const uint16_t*)X;
  g.T = p->T;
  g.tok = tok;
  g.alpha = alpha;
  g.W1 = (const uint16_t*)W1;
  g.W2 = (const uint16_t*)W2;
  g.H = (uint16_t*)H;
  g.Phi = (uint16_t*)Phi;
  g.Y = (uint16_t*)Y;
  g.row_off = seg_off_d;
  g.E = p->E;
  g.D = p->D;
  g.F = p->F;
  g.ntn = (int)ceil_div(p->F, 128);
  fwd_fc1_kernel<<<(unsigned)(mtiles * g.ntn), CfgW::NTHR, 0, s>>>(g);
  g.ntn = (int)ceil_div(p->D, BN);
  fwd_fc2_kernel<<<(unsigned)(mtiles * g.ntn), CfgW::NTHR, 0, s>>>(g);
  return launch_status();
}

size_t gemm_ws_bytes(const lrmoe_problem* p, const int64_t* row_off_h) {
  if (p->dtype != LRMOE_BF16) return 0;
  const WgradLayout L = wgrad_layout(p, row_off_h, wgrad_schedule(p, row_off_h).kc_max);
  return L.plan_bytes + L.partial_bytes;
}

lrmoe_status launch_grouped_gemm_bwd(const lrmoe_problem* p, const int64_t* row_off_h,
                                     const int64_t* row_off_d, const void* Dlt, const void* PhiC,
                                     const void* XC, const void* HC, const int32_t* hc_rows,
                                     const int32_t* phi_rows, const int32_t* x_rows, const int32_t* dlt_rows,
                                     const float* alpha, const void* W2, const void* W1,
                                     float* dW2, float* dW1, void* dH, void* dIn, int accumulate,
                                     void* ws, hipStream_t s, hipEvent_t din_ready) {
  const int E = p->E, D = p->D, F = p->F;
  // dIn is complete once the data-gradient launches are; the weight gradients follow
  auto mark_din = [&]() -> lrmoe_status {
    if (din_ready == nullptr) return LRMOE_OK;
    return hipEventRecord(din_ready, s) == hipSuccess ? LRMOE_OK : LRMOE_ERR_HIP;
  };
  const int64_t rows = row_off_h[E];
  // rows of the (possibly gathered) saved matrices: pair rows or token rows when mapped
  const int64_t hc_nrows = hc_rows ? p->N : rows, phi_nrows = phi_rows ? p->N : rows;
  const int64_t x_nrows = x_rows ? (int64_t)p->T : rows;
  // gradient rows read by token (dlt_rows: a token per packed row) from G [T x D]
  const int64_t dlt_nrows = dlt_rows ? (int64_t)p->T : rows;
  if (p->dtype == LRMOE_F32) {
    const float* dl = (const float*)Dlt;
    if (p->swiglu) {
      if (rows > 0) {
        f32_dgrad_kernel<EPI_SWIGLU><<<dim3((unsigned)rows, (unsigned)ceil_div(F, kAuxThr)), kAuxThr, 0, s>>>(
            dl, D, dlt_rows, dlt_nrows, alpha, (const float*)W2, D, (int64_t)F * D, F, D, row_off_d, E,
            (const float*)HC, hc_rows, hc_nrows, (float*)dH, 2 * F, F);
        f32_dgrad_kernel<EPI_STORE><<<dim3((unsigned)rows, (unsigned)ceil_div(D, kAuxThr)), kAuxThr, 0, s>>>(
            (const float*)dH, 2 * F, nullptr, 0, nullptr, (const float*)W1, 2 * F, (int64_t)D * 2 * F, D, 2 * F,
            row_off_d, E, nullptr, nullptr, 0, (float*)dIn, D, F);
      }
      if (mark_din() != LRMOE_OK) return LRMOE_ERR_HIP;
      if (E > 0) {
        f32_wgrad_kernel<<<dim3((unsigned)ceil_div(D, kAuxThr), F, E), kAuxThr, 0, s>>>(
            (const float*)PhiC, F, phi_rows, phi_nrows, dl, D, dlt_rows, dlt_nrows, F, D, row_off_d, dW2, accumulate);
        f32_wgrad_kernel<<<dim3((unsigned)ceil_div(2 * F, kAuxThr), D, E), kAuxThr, 0, s>>>(
            (const float*)XC, D, x_rows, x_nrows, (const float*)dH, 2 * F, nullptr, 0, D, 2 * F, row_off_d, dW1,
            accumulate);
      }
    } else {
      if (rows > 0)
        f32_dgrad_kernel<EPI_STORE><<<dim3((unsigned)rows, (unsigned)ceil_div(F, kAuxThr)), kAuxThr, 0, s>>>(
            dl, D, dlt_rows, dlt_nrows, alpha, (const float*)W2, D, (int64_t)F * D, F, D, row_off_d, E, nullptr,
            hc_rows, hc_nrows, (float*)dIn, F, F);
      if (mark_din() != LRMOE_OK) return LRMOE_ERR_HIP;
      if (E > 0)
        f32_wgrad_kernel<<<dim3((unsigned)ceil_div(D, kAuxThr), F, E), kAuxThr, 0, s>>>(
            (const float*)PhiC, F, phi_rows, phi_nrows, dl, D, dlt_rows, dlt_nrows, F, D, row_off_d, dW2, accumulate);
    }
    return launch_status();
  }

  // bf16 MFMA path
  int64_t mtiles = 0;
  for (int e = 0; e < E; ++e) mtiles += ceil_div(row_off_h[e + 1] - row_off_h[e], BM);
  DgradArgs d2{};
  d2.A = (const uint16_t*)Dlt;
  d2.lda = D;
  d2.a_rows = dlt_rows;
  d2.a_nrows = dlt_nrows;
  d2.alpha = alpha;
  d2.hc_rows = hc_rows;  // the pairs of the routing weights (and of HC's rows)
  d2.hc_nrows = hc_nrows;
  d2.W = (const uint16_t*)W2;
  d2.ldw = D;
  d2.w_estride = (int64_t)F * D;
  d2.N = F;
  d2.K = D;
  d2.ntn = (int)ceil_div(F, CfgD::BN);
  d2.row_off = row_off_d;
  d2.E = E;
  d2.F = F;
  if (p->swiglu) {
    d2.HC = (const uint16_t*)HC;
    d2.out = (uint16_t*)dH;
    d2.ldo = 2 * F;
    if (mtiles > 0) dgrad_kernel<EPI_SWIGLU><<<(unsigned)(mtiles * d2.ntn), CfgD::NTHR, 0, s>>>(d2);
    DgradArgs d1 = d2;
    d1.A = (const uint16_t*)dH;
    d1.lda = 2 * F;
    d1.a_rows = nullptr;
    d1.alpha = nullptr;
    d1.W = (const uint16_t*)W1;
    d1.ldw = 2 * F;
    d1.w_estride = (int64_t)D * 2 * F;
    d1.N = D;
    d1.K = 2 * F;
    d1.ntn = (int)ceil_div(D, CfgD::BN);
    d1.HC = nullptr;
    d1.hc_rows = nullptr;
    d1.out = (uint16_t*)dIn;
    d1.ldo = D;
    if (mtiles > 0) dgrad_kernel<EPI_STORE><<<(unsigned)(mtiles * d1.ntn), CfgD::NTHR, 0, s>>>(d1);
  } else {
    d2.out = (uint16_t*)dIn;
    d2.ldo = F;
    if (mtiles > 0) dgrad_kernel<EPI_STORE><<<(unsigned)(mtiles * d2.ntn), CfgD::NTHR, 0, s>>>(d2);
  }
  if (mark_din() != LRMOE_OK) return LRMOE_ERR_HIP;

  const WgradSchedule sched = wgrad_schedule(p, row_off_h);
  const WgradLayout L = wgrad_layout(p, row_off_h, sched.kc_max);
  WgradArgs w{};
  w.t[0] = WgradType{(const uint16_t*)PhiC, F, phi_rows, phi_nrows, (const uint16_t*)Dlt, D, dW2, F, D,
                     (int)ceil_div(F, BM), (int)ceil_div(D, BN), wgrad_tiles(F, D), dlt_rows, dlt_nrows};
  w.ntypes = 1;
  if (p->swiglu) {
    w.t[1] = WgradType{(const uint16_t*)XC, D, x_rows, x_nrows, (const uint16_t*)dH, 2 * F, dW1, D, 2 * F,
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
  w.kc_max = sched.kc_max;
  for (int x = 0; x < 9; ++x) w.xlo[x] = sched.xlo[x];
  if (E > 0) {
    const int64_t per_xcd = sched.per_xcd;
    wgrad_plan_kernel<<<1, kAuxThr, 0, s>>>(w);
    const unsigned grid = (unsigned)(8 * per_xcd);
    const bool g0 = phi_rows != nullptr, g1 = x_rows != nullptr, gb0 = dlt_rows != nullptr;
    if (per_xcd > 0) {
      if (gb0 && g1) wgrad_kernel<false, true, true><<<grid, CfgW::NTHR, 0, s>>>(w);
      else if (gb0) wgrad_kernel<false, false, true><<<grid, CfgW::NTHR, 0, s>>>(w);
      else if (g0 && g1) wgrad_kernel<true, true, false><<<grid, CfgW::NTHR, 0, s>>>(w);
      else if (g0) wgrad_kernel<true, false, false><<<grid, CfgW::NTHR, 0, s>>>(w);
      else if (g1) wgrad_kernel<false, true, false><<<grid, CfgW::NTHR, 0, s>>>(w);
      else wgrad_kernel<false, false, false><<<grid, CfgW::NTHR, 0, s>>>(w);
    }
    if (L.nreduce > 0) wgrad_reduce_kernel<<<(unsigned)(L.nreduce * kRedParts), kAuxThr, 0, s>>>(w);
  }
  return launch_status();
}

}  // namespace lrmoe
