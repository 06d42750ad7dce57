// Step 2: per-expert TopK under fixed quotas (LRMoE paper, section 3.3 and appendix 7.2,
// Proposition 7.1: inside one partition, keeping the q largest scores maximises the
// retained calibration value). Each expert segment keeps its q_e largest scores; equal
// scores at the threshold go to the lower pair index, and the retained indices come out
// in ascending order (the packing order of the compact buffers).
//
// Scores are non-negative f32, so their bit patterns order like unsigned integers. The
// q_e-th largest key of every segment is found by a three-pass most-significant-digit
// radix select (11, 11 and 10 bits). Every pass is one launch over (chunk, expert)
// blocks: blocks build LDS histograms of the digit among keys that still match the
// prefix, add them to a global per-expert histogram, and the last block to finish (an
// atomic ticket) walks each histogram from the top to fix the next digit. Two more
// launches count, per chunk, keys above and equal to the threshold, then write the
// retained indices at positions given by block-level ballot scans. Nothing spins: each
// block either does its share and leaves or, being last, finishes the pass.
#include "common.h"

namespace lrmoe {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;
constexpr int kChunk = kSelThreads * kSelPer;  // keys per block
constexpr int kBins = 2048;

enum : uint32_t { kKeepNone = 0, kKeepAll = 1, kKeepThreshold = 2 };

struct SegState {
  uint32_t prefix;  // digits fixed so far (after the last pass: the threshold key)
  uint32_t mask;    // bits of prefix that are fixed
  uint32_t need;    // rank still to find among keys matching prefix (ties kept at the end)
  uint32_t cnt_gt;  // keys strictly above the prefix range
  uint32_t mode;
  uint32_t pad[3];
};

struct SelWs {
  uint32_t* hist;    // [E][kBins]
  SegState* state;   // [E]
  uint32_t* counts;  // [E][maxch][2]  keys above / equal to the threshold, per chunk
  uint32_t* offs;    // [E][maxch][2]  exclusive prefix of counts within the segment
  uint32_t* ticket;  // [1]
};

int max_chunks(const lrmoe_problem* p) {
  int64_t m = 1;
  for (int e = 0; e < p->E; ++e) m = std::max<int64_t>(m, ceil_div(p->seg_off[e + 1] - p->seg_off[e], kChunk));
  return (int)m;
}

SelWs carve(void* ws, int E, int maxch) {
  char* b = (char*)ws;
  SelWs w;
  size_t o = 0;
  w.hist = (uint32_t*)(b + o);
  o = align_up(o + sizeof(uint32_t) * (size_t)E * kBins, 256);
  w.state = (SegState*)(b + o);
  o = align_up(o + sizeof(SegState) * (size_t)E, 256);
  w.counts = (uint32_t*)(b + o);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  w.offs = (uint32_t*)(b + o);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  w.ticket = (uint32_t*)(b + o);
  return w;
}

size_t carve_bytes(int E, int maxch) {
  size_t o = 0;
  o = align_up(o + sizeof(uint32_t) * (size_t)E * kBins, 256);
  o = align_up(o + sizeof(SegState) * (size_t)E, 256);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  return o + 256;
}

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in every thread of the block that finished last among all blocks of the grid.
__device__ __forceinline__ bool last_block_done(uint32_t* ticket) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t total = gridDim.x * gridDim.y;
    const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (t == total - 1);
  }
  __syncthreads();
  if (s_last) __threadfence();
  return s_last != 0;
}

__global__ __launch_bounds__(kSelThreads) void select_init_kernel(int E, const int64_t* __restrict__ seg_off,
                                                                  const int32_t* __restrict__ quota,
                                                                  SelWs w) {
  const int64_t gid = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
  if (gid < (int64_t)E * kBins) w.hist[gid] = 0;
  if (gid < E) {
    const int64_t n = seg_off[gid + 1] - seg_off[gid];
    const int64_t q = quota[gid];
    SegState s;
    s.prefix = 0;
    s.mask = 0;
    s.need = (uint32_t)q;
    s.cnt_gt = 0;
    s.mode = q <= 0 ? kKeepNone : (q >= n ? kKeepAll : kKeepThreshold);
    s.pad[0] = s.pad[1] = s.pad[2] = 0;
    w.state[gid] = s;
  }
  if (gid == 0) *w.ticket = 0;
}

__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(int shift, int nbits, const float* __restrict__ R,
                                                                  const int64_t* __restrict__ seg_off,
                                                                  SelWs w, int E) {
  __shared__ uint32_t h[kBins];
  const int e = blockIdx.y, tid = threadIdx.x;
  const SegState st = w.state[e];
  const int64_t lo = seg_off[e] + (int64_t)blockIdx.x * kChunk;
  const int64_t hi = min(seg_off[e + 1], lo + kChunk);
  const uint32_t nb = 1u << nbits;
  if (st.mode == kKeepThreshold && lo < hi) {  // uniform across the block
    for (uint32_t b = tid; b < nb; b += kSelThreads) h[b] = 0;
    __syncthreads();
    for (int64_t i = lo + tid; i < hi; i += kSelThreads) {
      const uint32_t key = __float_as_uint(R[i]);
      if ((key & st.mask) == st.prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    for (uint32_t b = tid; b < nb; b += kSelThreads) {
      const uint32_t c = h[b];
      if (c) atomicAdd(&w.hist[(size_t)e * kBins + b], c);
    }
  }
  if (!last_block_done(w.ticket)) return;

  // Last block: fix this pass's digit of every thresholded segment, one wavefront each.
  const int wave = tid / kWave, lane = tid % kWave;
  const uint32_t per = nb / kWave;  // bins per lane; lane 0 owns the highest bins
  for (int e2 = wave; e2 < E; e2 += kSelThreads / kWave) {
    SegState s2 = w.state[e2];
    if (s2.mode != kKeepThreshold) continue;
    uint32_t* hg = w.hist + (size_t)e2 * kBins;
    const int top = (int)(nb - lane * per);
    uint32_t c = 0;
    for (int b = top - (int)per; b < top; ++b) c += load_agent(&hg[b]);
    uint32_t inc = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += v;
    }
    const uint32_t exc = inc - c;
    const bool mine = exc < s2.need && inc >= s2.need;
    if (mine) {
      uint32_t above = exc;
      int b = top - 1;
      for (; b > top - (int)per; --b) {
        const uint32_t cb = load_agent(&hg[b]);
        if (above + cb >= s2.need) break;
        above += cb;
      }
      s2.need -= above;
      s2.cnt_gt += above;
      s2.prefix |= (uint32_t)b << shift;
      s2.mask |= (nb - 1) << shift;
      w.state[e2] = s2;
    }
    for (uint32_t b = lane; b < nb; b += kWave) hg[b] = 0;  // ready for the next pass
  }
  __syncthreads();
  if (tid == 0) *w.ticket = 0;
}

__global__ __launch_bounds__(kSelThreads) void select_count_kernel(const float* __restrict__ R,
                                                                   const int64_t* __restrict__ seg_off,
                                                                   SelWs w, int E, int maxch) {
  __shared__ uint32_t red[2][kSelThreads / kWave];
  const int e = blockIdx.y, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const SegState st = w.state[e];
  const int64_t lo = seg_off[e] + (int64_t)blockIdx.x * kChunk;
  const int64_t hi = min(seg_off[e + 1], lo + kChunk);
  uint32_t gt = 0, eq = 0;
  if (st.mode != kKeepNone) {
    for (int64_t i = lo + tid; i < hi; i += kSelThreads) {
      const uint32_t key = __float_as_uint(R[i]);
      gt += (st.mode == kKeepAll || key > st.prefix) ? 1u : 0u;
      eq += (st.mode == kKeepThreshold && key == st.prefix) ? 1u : 0u;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt += __shfl_xor(gt, o, kWave);
    eq += __shfl_xor(eq, o, kWave);
  }
  if (lane == 0) {
    red[0][wave] = gt;
    red[1][wave] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0, b = 0;
    for (int i = 0; i < kSelThreads / kWave; ++i) {
      a += red[0][i];
      b += red[1][i];
    }
    const size_t slot = ((size_t)e * maxch + blockIdx.x) * 2;
    w.counts[slot] = a;
    w.counts[slot + 1] = b;
  }
  if (!last_block_done(w.ticket)) return;
  for (int e2 = tid; e2 < E; e2 += kSelThreads) {
    const int64_t n = seg_off[e2 + 1] - seg_off[e2];
    const int nch = (int)((n + kChunk - 1) / kChunk);
    uint32_t rg = 0, re = 0;
    for (int c = 0; c < nch && c < maxch; ++c) {
      const size_t slot = ((size_t)e2 * maxch + c) * 2;
      w.offs[slot] = rg;
      w.offs[slot + 1] = re;
      rg += load_agent(&w.counts[slot]);
      re += load_agent(&w.counts[slot + 1]);
    }
  }
  __syncthreads();
  if (tid == 0) *w.ticket = 0;
}

__global__ __launch_bounds__(kSelThreads) void select_write_kernel(const float* __restrict__ R,
                                                                   const int64_t* __restrict__ seg_off,
                                                                   const int64_t* __restrict__ cseg_off,
                                                                   SelWs w, int maxch, int64_t K_tot,
                                                                   int32_t* __restrict__ sel,
                                                                   uint8_t* __restrict__ keep) {
  __shared__ uint32_t wtot[2][2][kSelThreads / kWave];
  const int e = blockIdx.y, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const SegState st = w.state[e];
  const int64_t lo = seg_off[e] + (int64_t)blockIdx.x * kChunk;
  const int64_t hi = min(seg_off[e + 1], lo + kChunk);
  if (lo >= hi) return;  // uniform across the block
  const size_t slot = ((size_t)e * maxch + blockIdx.x) * 2;
  const uint32_t base_gt = w.offs[slot], base_eq = w.offs[slot + 1];
  const uint32_t need = st.mode == kKeepThreshold ? st.need : 0u;
  const int64_t cbase = cseg_off[e], cend = min(cseg_off[e + 1], K_tot);
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t run_gt = 0, run_eq = 0;
  for (int r = 0; r < kSelPer; ++r) {
    const int64_t i = lo + (int64_t)r * kSelThreads + tid;
    const bool valid = i < hi;
    const uint32_t key = valid ? __float_as_uint(R[i]) : 0u;
    const bool gt = valid && (st.mode == kKeepAll || (st.mode == kKeepThreshold && key > st.prefix));
    const bool eq = valid && st.mode == kKeepThreshold && key == st.prefix;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int buf = r & 1;
    if (lane == 0) {
      wtot[buf][0][wave] = (uint32_t)__popcll(bg);
      wtot[buf][1][wave] = (uint32_t)__popcll(be);
    }
    __syncthreads();
    uint32_t og = 0, oe = 0, tg = 0, te = 0;
#pragma unroll
    for (int v = 0; v < kSelThreads / kWave; ++v) {
      const uint32_t a = wtot[buf][0][v], b = wtot[buf][1][v];
      if (v < wave) {
        og += a;
        oe += b;
      }
      tg += a;
      te += b;
    }
    const uint32_t gt_before = base_gt + run_gt + og + (uint32_t)__popcll(bg & lt_mask);
    const uint32_t eq_before = base_eq + run_eq + oe + (uint32_t)__popcll(be & lt_mask);
    const bool k = gt || (eq && eq_before < need);
    if (k) {
      const int64_t pos = cbase + gt_before + min(eq_before, need);
      if (pos < cend) sel[pos] = (int32_t)i;
    }
    if (keep != nullptr && valid) keep[i] = k ? 1 : 0;
    run_gt += tg;
    run_eq += te;
  }
}

}  // namespace

size_t select_ws_bytes(const lrmoe_problem* p) { return carve_bytes(p->E, max_chunks(p)); }

lrmoe_status launch_select(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                           const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel,
                           uint8_t* keep, void* ws, hipStream_t s) {
  const int E = p->E, maxch = max_chunks(p);
  int64_t K_tot = 0;
  for (int e = 0; e < E; ++e) K_tot += p->quota[e];
  SelWs w = carve(ws, E, maxch);
  const int64_t init_threads = std::max<int64_t>((int64_t)E * kBins, 1);
  select_init_kernel<<<(unsigned)ceil_div(init_threads, kSelThreads), kSelThreads, 0, s>>>(E, seg_off_d, quota_d, w);
  dim3 grid(maxch, E);
  select_hist_kernel<<<grid, kSelThreads, 0, s>>>(21, 11, R, seg_off_d, w, E);
  select_hist_kernel<<<grid, kSelThreads, 0, s>>>(10, 11, R, seg_off_d, w, E);
  select_hist_kernel<<<grid, kSelThreads, 0, s>>>(0, 10, R, seg_off_d, w, E);
  select_count_kernel<<<grid, kSelThreads, 0, s>>>(R, seg_off_d, w, E, maxch);
  select_write_kernel<<<grid, kSelThreads, 0, s>>>(R, seg_off_d, cseg_off_d, w, maxch, K_tot, sel, keep);
  return launch_status();
}

}  // namespace lrmoe
