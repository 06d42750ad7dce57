// Step 2: per-expert TopK under fixed quotas (LRMoE paper, section 3.3 and appendix 7.2,
// Proposition 7.1: inside one partition, keeping the q largest scores maximises the
// retained calibration value). Each expert segment keeps its q_e largest scores; equal
// scores at the threshold go to the lower pair index, and the retained indices come out
// in ascending order (the packing order of the compact buffers).
//
// Scores are non-negative f32, so their bit patterns order like unsigned integers. The
// q_e-th largest key of every segment is found by a three-pass most-significant-digit
// radix select (11, 11 and 10 bits). In pass p, chunk blocks (4096 keys of one segment
// each) build LDS histograms of the digit among keys that still match the prefix fixed so
// far and add them to the segment's global histogram of that pass (each pass has its own).
// The digit of pass p is fixed in the next launch, by every one of its blocks: each scans
// the finished histogram from the highest bin (a few KB from L2) and block 0 of the segment
// records the resulting state for the launches after it. The write side is two launches:
// chunk blocks count keys above and equal to the threshold (fixing the last digit first),
// and chunk blocks write the retained indices at positions given by the counts of the
// chunks before them and block-level ballot scans (segments of more than 256 chunks get
// those offsets from a launch of their own). Kernel boundaries order every step, so no
// block waits on another and no block needs a device-wide fence. On request the write
// launch also records, for every retained pair, its packed row in a (token, slot) map and
// its token and slot in packed order (the init launch clears the map), so compaction and
// the scatter need no map of their own.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace lrmoe {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;
constexpr int kChunk = kSelThreads * kSelPer;  // keys per chunk block
constexpr int kBins = 2048;
constexpr int kPasses = 3;
constexpr int kShift[kPasses] = {21, 10, 0}, kBits[kPasses] = {11, 11, 10};
constexpr int kPassBins = (1 << 11) + (1 << 11) + (1 << 10);  // histogram bins of all passes
// segments of at most this many chunks get their write offsets inside the write launch
constexpr int kFusedOffsMaxChunks = kSelThreads;

enum : uint32_t { kKeepNone = 0, kKeepAll = 1, kKeepThreshold = 2 };

struct SegState {
  uint32_t prefix;  // digits fixed so far (after the last pass: the threshold key)
  uint32_t mask;    // bits of prefix that are fixed
  uint32_t need;    // rank still to find among keys matching prefix (ties kept at the end)
  uint32_t mode;
};

// Optional outputs of the write kernel: for every retained pair j at packed row c, its
// token and slot (ctok[c], cslot[c]; -1 for both when either is out of range) and the
// (token, slot) -> packed row map entry pmap[tok * K + slot] = c.
struct PosOut {
  const int32_t* tok;
  const int32_t* slot;
  int32_t* pmap;  // [T x K] or nullptr
  int32_t* ctok;
  int32_t* cslot;
  int T, K;
};

struct SelWs {
  uint32_t* hist;    // [E][kPassBins]: pass 0 bins, then pass 1, then pass 2
  SegState* state;   // [kPasses + 1][E]: state[p] holds the digits of passes < p
  uint32_t* counts;  // [E][maxch][2]  keys above / equal to the threshold, per chunk
  uint32_t* offs;    // [E][maxch][2]  exclusive prefix of counts within the segment
};

__host__ __device__ constexpr int pass_bin0(int pass) { return pass == 0 ? 0 : pass == 1 ? 2048 : 4096; }

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
  o = align_up(o + sizeof(uint32_t) * (size_t)E * kPassBins, 256);
  w.state = (SegState*)(b + o);
  o = align_up(o + sizeof(SegState) * (size_t)E * (kPasses + 1), 256);
  w.counts = (uint32_t*)(b + o);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  w.offs = (uint32_t*)(b + o);
  return w;
}

size_t carve_bytes(int E, int maxch) {
  size_t o = 0;
  o = align_up(o + sizeof(uint32_t) * (size_t)E * kPassBins, 256);
  o = align_up(o + sizeof(SegState) * (size_t)E * (kPasses + 1), 256);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  o = align_up(o + sizeof(uint32_t) * 2 * (size_t)E * maxch, 256);
  return o;
}

// Keys of the chunk block at [lo, hi): thread t holds keys lo + r*256 + t, r < kSelPer,
// all loaded before any is used. Bit r of the result marks keys inside the chunk.
__device__ __forceinline__ uint32_t load_chunk(const float* __restrict__ R, int64_t lo, int64_t hi,
                                               uint32_t (&k)[kSelPer]) {
  uint32_t ok = 0;
#pragma unroll
  for (int r = 0; r < kSelPer; ++r) {
    const int64_t i = lo + (int64_t)r * kSelThreads + threadIdx.x;
    k[r] = i < hi ? __float_as_uint(R[i]) : 0u;
    ok |= (i < hi ? 1u : 0u) << r;
  }
  return ok;
}

__global__ __launch_bounds__(kSelThreads) void select_init_kernel(int E, const int64_t* __restrict__ seg_off,
                                                                  const int32_t* __restrict__ quota,
                                                                  SelWs w, int64_t positions,
                                                                  int32_t* __restrict__ pmap) {
  const int64_t gid = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
  if (gid < (int64_t)E * kPassBins) w.hist[gid] = 0;
  if (pmap != nullptr && gid < positions) pmap[gid] = -1;  // positions with no retained pair
  if (gid < E) {
    const int64_t n = seg_off[gid + 1] - seg_off[gid];
    const int64_t q = quota[gid];
    SegState s;
    s.prefix = 0;
    s.mask = 0;
    s.need = (uint32_t)q;
    s.mode = q <= 0 ? kKeepNone : (q >= n ? kKeepAll : kKeepThreshold);
    w.state[gid] = s;
  }
}

// Block-wide inclusive prefix in thread order (256 threads); total in tot. Every thread of
// the block must call it.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t& tot, uint32_t* sh) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  uint32_t pre = 0;
  tot = 0;
#pragma unroll
  for (int v2 = 0; v2 < kSelThreads / kWave; ++v2) {
    if (v2 < wave) pre += sh[v2];
    tot += sh[v2];
  }
  __syncthreads();
  return pre + inc;
}

// Fixes the digit of pass `pass` from the segment's finished histogram of that pass
// (thread t scans the `per` bins just below nb - per*t, thread 0 the highest): the rank
// still needed falls in exactly one bin. Every thread of the block calls it and gets the new
// state; `sh` and `out` are the block's shared scratch.
__device__ __forceinline__ SegState fix_digit(const uint32_t* __restrict__ hseg, int pass, SegState st, uint32_t* sh,
                                              SegState* out) {
  const int tid = threadIdx.x, shift = kShift[pass];
  const uint32_t nb = 1u << kBits[pass], per = nb / kSelThreads;  // 8 or 4
  const uint32_t* hg = hseg + pass_bin0(pass);
  const int top = (int)(nb - tid * per);
  uint32_t c[8];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[j] = j < (int)per ? hg[top - 1 - j] : 0u;  // c[0] is the thread's highest bin
    sum += c[j];
  }
  if (tid == 0) *out = st;
  uint32_t tot;
  const uint32_t inc = block_incl_scan(sum, tot, sh);
  const uint32_t exc = inc - sum;
  if (exc < st.need && inc >= st.need) {  // exactly one thread
    uint32_t above = exc;
    int j = 0;
    for (; j < (int)per - 1; ++j) {
      if (above + c[j] >= st.need) break;
      above += c[j];
    }
    SegState ns = st;
    ns.need -= above;
    ns.prefix |= (uint32_t)(top - 1 - j) << shift;
    ns.mask |= (nb - 1) << shift;
    *out = ns;
  }
  __syncthreads();
  return *out;
}

// The state after passes < p, for a block of the launch that needs it: pass 0's comes from
// the init launch; later ones are fixed here from pass p-1's histogram on top of the state
// the previous launch recorded, and block 0 of the segment records them for the next launch.
__device__ __forceinline__ SegState state_before(const SelWs& w, int E, int e, int p, bool needed, uint32_t* sh,
                                                 SegState* out) {
  SegState st = w.state[(size_t)(p > 0 ? p - 1 : 0) * E + e];
  if (p > 0 && st.mode == kKeepThreshold && (needed || blockIdx.x == 0))  // uniform across the block
    st = fix_digit(w.hist + (size_t)e * kPassBins, p - 1, st, sh, out);
  if (p > 0 && blockIdx.x == 0 && threadIdx.x == 0) w.state[(size_t)p * E + e] = st;
  return st;
}

__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(int pass, const float* __restrict__ R,
                                                                  const int64_t* __restrict__ seg_off, SelWs w, int E) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t sh[kSelThreads / kWave];
  __shared__ SegState out;
  const int e = blockIdx.y, tid = threadIdx.x;
  const int64_t lo = seg_off[e] + (int64_t)blockIdx.x * kChunk;
  const int64_t hi = min(seg_off[e + 1], lo + kChunk);
  const SegState st = state_before(w, E, e, pass, lo < hi, sh, &out);
  if (st.mode != kKeepThreshold || lo >= hi) return;  // uniform across the block
  const int shift = kShift[pass];
  const uint32_t nb = 1u << kBits[pass];
  uint32_t k[kSelPer];
  const uint32_t ok = load_chunk(R, lo, hi, k);
  for (uint32_t b = tid; b < nb; b += kSelThreads) h[b] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSelPer; ++r)
    if ((ok >> r & 1) && (k[r] & st.mask) == st.prefix) atomicAdd(&h[(k[r] >> shift) & (nb - 1)], 1u);
  __syncthreads();
  uint32_t* hg = w.hist + (size_t)e * kPassBins + pass_bin0(pass);
  for (uint32_t b = tid; b < nb; b += kSelThreads) {
    const uint32_t c = h[b];
    if (c) atomicAdd(&hg[b], c);
  }
}

__global__ __launch_bounds__(kSelThreads) void select_count_kernel(const float* __restrict__ R,
                                                                   const int64_t* __restrict__ seg_off,
                                                                   SelWs w, int maxch, int E) {
  __shared__ uint32_t red[2][kSelThreads / kWave];
  __shared__ uint32_t sh[kSelThreads / kWave];
  __shared__ SegState out;
  const int e = blockIdx.y, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t lo = seg_off[e] + (int64_t)blockIdx.x * kChunk;
  const int64_t hi = min(seg_off[e + 1], lo + kChunk);
  const SegState st = state_before(w, E, e, kPasses, lo < hi, sh, &out);  // the threshold key
  if (lo >= hi) return;  // uniform across the block
  uint32_t gt = 0, eq = 0;
  if (st.mode != kKeepNone) {
    uint32_t k[kSelPer];
    const uint32_t ok = load_chunk(R, lo, hi, k);
#pragma unroll
    for (int r = 0; r < kSelPer; ++r) {
      const bool v = ok >> r & 1;
      gt += (v && (st.mode == kKeepAll || k[r] > st.prefix)) ? 1u : 0u;
      eq += (v && st.mode == kKeepThreshold && k[r] == st.prefix) ? 1u : 0u;
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
}

// One block per segment: exclusive prefix of its per-chunk counts, 256 chunks at a time.
__global__ __launch_bounds__(kSelThreads) void select_offs_kernel(const int64_t* __restrict__ seg_off, SelWs w,
                                                                  int maxch) {
  __shared__ uint32_t sh[2][kSelThreads / kWave];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int64_t n = seg_off[e + 1] - seg_off[e];
  const int nch = (int)min<int64_t>((n + kChunk - 1) / kChunk, maxch);
  uint32_t rg = 0, re = 0;
  for (int c0 = 0; c0 < nch; c0 += kSelThreads) {  // uniform trip count
    const int c = c0 + tid;
    const size_t slot = ((size_t)e * maxch + c) * 2;
    const uint32_t g = c < nch ? w.counts[slot] : 0u, q = c < nch ? w.counts[slot + 1] : 0u;
    uint32_t tg, tq;
    const uint32_t ig = block_incl_scan(g, tg, sh[0]);
    const uint32_t iq = block_incl_scan(q, tq, sh[1]);
    if (c < nch) {
      w.offs[slot] = rg + ig - g;
      w.offs[slot + 1] = re + iq - q;
    }
    rg += tg;
    re += tq;
  }
}

__global__ __launch_bounds__(kSelThreads) void select_write_kernel(const float* __restrict__ R,
                                                                   const int64_t* __restrict__ seg_off,
                                                                   const int64_t* __restrict__ cseg_off,
                                                                   SelWs w, int maxch, int E, bool fused_offs,
                                                                   int64_t K_tot, int32_t* __restrict__ sel,
                                                                   uint8_t* __restrict__ keep, PosOut po) {
  __shared__ uint32_t wtot[kSelPer][2][kSelThreads / kWave];
  __shared__ uint32_t sh[2][kSelThreads / kWave];
  const int e = blockIdx.y, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const SegState st = w.state[(size_t)kPasses * E + e];
  const int64_t lo = seg_off[e] + (int64_t)blockIdx.x * kChunk;
  const int64_t hi = min(seg_off[e + 1], lo + kChunk);
  if (lo >= hi) return;  // uniform across the block
  uint32_t base_gt, base_eq;
  if (fused_offs) {  // uniform: the counts of the segment's chunks before this one (fewer than 256)
    const int c = tid;
    const size_t cs = ((size_t)e * maxch + c) * 2;
    const bool before = c < (int)blockIdx.x;
    const uint32_t g = before ? w.counts[cs] : 0u, q = before ? w.counts[cs + 1] : 0u;
    uint32_t tg, tq;
    block_incl_scan(g, tg, sh[0]);
    block_incl_scan(q, tq, sh[1]);
    base_gt = tg;
    base_eq = tq;
  } else {
    const size_t slot = ((size_t)e * maxch + blockIdx.x) * 2;
    base_gt = w.offs[slot];
    base_eq = w.offs[slot + 1];
  }
  const uint32_t need = st.mode == kKeepThreshold ? st.need : 0u;
  const int64_t cbase = cseg_off[e], cend = min(cseg_off[e + 1], K_tot);
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t k[kSelPer];
  const uint32_t ok = load_chunk(R, lo, hi, k);
  // the pairs' tokens and slots (with the map only), all loaded before any is used, as the keys
  int32_t pt[kSelPer], ps[kSelPer];
  if (po.pmap != nullptr) {  // uniform
#pragma unroll
    for (int r = 0; r < kSelPer; ++r) {
      const int64_t i = lo + (int64_t)r * kSelThreads + tid;
      pt[r] = i < hi ? po.tok[i] : -1;
      ps[r] = i < hi ? po.slot[i] : -1;
    }
  }
  uint64_t bg[kSelPer], be[kSelPer];
#pragma unroll
  for (int r = 0; r < kSelPer; ++r) {
    const bool v = ok >> r & 1;
    const bool gt = v && (st.mode == kKeepAll || (st.mode == kKeepThreshold && k[r] > st.prefix));
    const bool eq = v && st.mode == kKeepThreshold && k[r] == st.prefix;
    bg[r] = __ballot(gt);
    be[r] = __ballot(eq);
    if (lane == 0) {
      wtot[r][0][wave] = (uint32_t)__popcll(bg[r]);
      wtot[r][1][wave] = (uint32_t)__popcll(be[r]);
    }
  }
  __syncthreads();
  // keys before (r, wave, lane) in index order: rows r' < r, then earlier waves of row r
  uint32_t run_gt = 0, run_eq = 0;
#pragma unroll
  for (int r = 0; r < kSelPer; ++r) {
    uint32_t og = 0, oe = 0, tg = 0, te = 0;
#pragma unroll
    for (int v = 0; v < kSelThreads / kWave; ++v) {
      const uint32_t a = wtot[r][0][v], b = wtot[r][1][v];
      if (v < wave) {
        og += a;
        oe += b;
      }
      tg += a;
      te += b;
    }
    const int64_t i = lo + (int64_t)r * kSelThreads + tid;
    const bool gt = bg[r] >> lane & 1, eq = be[r] >> lane & 1;
    const uint32_t gt_before = base_gt + run_gt + og + (uint32_t)__popcll(bg[r] & lt_mask);
    const uint32_t eq_before = base_eq + run_eq + oe + (uint32_t)__popcll(be[r] & lt_mask);
    const bool kp = gt || (eq && eq_before < need);
    if (kp) {
      const int64_t pos = cbase + gt_before + min(eq_before, need);
      if (pos < cend) {
        sel[pos] = (int32_t)i;
        if (po.pmap != nullptr) {  // the packed row's token and slot, and its map entry
          const int t = pt[r], sl = ps[r];
          const bool valid = t >= 0 && t < po.T && sl >= 0 && sl < po.K;
          po.ctok[pos] = valid ? t : -1;
          po.cslot[pos] = valid ? sl : -1;
          if (valid) po.pmap[(int64_t)t * po.K + sl] = (int32_t)pos;
        }
      }
    }
    if (keep != nullptr && (ok >> r & 1)) keep[i] = kp ? 1 : 0;
    run_gt += tg;
    run_eq += te;
  }
}

}  // namespace

size_t select_ws_bytes(const lrmoe_problem* p) { return carve_bytes(p->E, max_chunks(p)); }

lrmoe_status launch_select(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                           const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel,
                           uint8_t* keep, const int32_t* tok, const int32_t* slot, int32_t* pmap,
                           int32_t* ctok, int32_t* cslot, void* ws, hipStream_t s) {
  const int E = p->E, maxch = max_chunks(p);
  if (E <= 0) return LRMOE_OK;
  int64_t K_tot = 0;
  for (int e = 0; e < E; ++e) K_tot += p->quota[e];
  SelWs w = carve(ws, E, maxch);
  const int64_t positions = pmap != nullptr ? (int64_t)p->T * p->K : 0;
  const PosOut po{tok, slot, pmap, ctok, cslot, p->T, p->K};
  const int64_t init_threads = std::max<int64_t>((int64_t)E * kPassBins, positions);
  select_init_kernel<<<(unsigned)ceil_div(init_threads, kSelThreads), kSelThreads, 0, s>>>(E, seg_off_d, quota_d, w,
                                                                                           positions, pmap);
  const dim3 grid(maxch, E);
  for (int pass = 0; pass < kPasses; ++pass)
    select_hist_kernel<<<grid, kSelThreads, 0, s>>>(pass, R, seg_off_d, w, E);
  select_count_kernel<<<grid, kSelThreads, 0, s>>>(R, seg_off_d, w, maxch, E);
  const bool fused_offs = maxch <= kFusedOffsMaxChunks;
  if (!fused_offs) select_offs_kernel<<<E, kSelThreads, 0, s>>>(seg_off_d, w, maxch);
  select_write_kernel<<<grid, kSelThreads, 0, s>>>(R, seg_off_d, cseg_off_d, w, maxch, E, fused_offs, K_tot, sel,
                                                   keep, po);
  return launch_status();
}

// ---------------------------------------------------------------- allocation-free variant

namespace {

// Scratch of the allocation-free selection (lrmoe_select_noalloc): a fixed array that every
// GPU the library runs on holds until the process ends. Host code never passes the array's
// name to a kernel: it is a host-side stand-in, not a device address. The device address is
// fetched once per device, with that device current, and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device).
lrmoe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LRMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LRMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LRMOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LRMOE_OK;
}

}  // namespace

size_t select_noalloc_max_bytes() { return kNoAllocScratchBytes; }

lrmoe_status launch_select_noalloc(const lrmoe_problem* p, const float* R, const int64_t* seg_off_d,
                                   const int32_t* quota_d, const int64_t* cseg_off_d, int32_t* sel, uint8_t* keep,
                                   const int32_t* tok, const int32_t* slot, int32_t* pmap, int32_t* ctok,
                                   int32_t* cslot, hipStream_t s) {
  if (select_ws_bytes(p) > kNoAllocScratchBytes) return LRMOE_ERR_WORKSPACE;
  void* ptr = nullptr;
  const lrmoe_status st = noalloc_scratch(&ptr);
  if (st != LRMOE_OK) return st;
  // the selection clears what it accumulates into (histograms, segment state) in its own
  // first launch, so the previous call's contents do no harm
  return launch_select(p, R, seg_off_d, quota_d, cseg_off_d, sel, keep, tok, slot, pmap, ctok, cslot, ptr, s);
}

}  // namespace lrmoe
