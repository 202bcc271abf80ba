// qsa_topk.hip -- selected ids of every (token, group) row.
//
// Pages: "round 6 track b - qsa flash" (delivered change: identity ids when
// the token sees at most 2051 cells, explicit selection above that, also
// inside chunks that cross the threshold; experiment contract: the selected-
// index semantics above budget are kept).  Tie rule and order (lower index
// first on equal scores, ids ascending) are this library's reading.
//
// One workgroup of 1024 threads per row.  Identity rows are written
// directly.  Above budget, an MSB-first radix select over order-preserving
// 32-bit keys finds the budget-th largest key K (4 passes of 8-bit digits,
// per-wave LDS histograms), then an ordered compaction writes, in ascending
// index order, every cell with key > K and the lowest-index cells with
// key == K until exactly `budget` ids are out.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Order-preserving key: larger float -> larger unsigned; -0.0 == +0.0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkShared {
  uint32_t hist[kTopkWaves][256];
  uint32_t tot[256];
  uint32_t wscan[kTopkWaves];
  uint32_t wscan2[kTopkWaves];
  uint32_t digit;
  uint32_t above;   // keys in digits strictly above the chosen one
  uint32_t in_dig;  // keys in the chosen digit
};

// Exclusive prefix of `flag` over the block in thread order; returns the
// thread's offset and writes the block total.  Two barriers.
__device__ __forceinline__ uint32_t block_excl_scan(bool flag, uint32_t* wsc, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsc[w] = __popcll(m);
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t c = wsc[i];
    off += (i < w) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return off + before;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int32_t* __restrict__ ids, int T,
                                                            int pos0, int G, int budget,
                                                            int64_t n_cells) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;  // t * G + g
  const int t = row / G;
  const int64_t n = (int64_t)pos0 + t + 1;
  int32_t* out = ids + (int64_t)row * budget;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  if (n <= budget) {
    for (int i = tid; i < budget; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const float* s = scores + (int64_t)row * n_cells;

  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)budget, eq_total = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = score_key(s[i]);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[w][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < kTopkWaves; ++i) c += sh.hist[i][tid];
      sh.tot[tid] = c;
    }
    __syncthreads();
    // digit d* with  above(d*) < krem <= above(d*) + tot[d*], scanning from
    // the top digit: inclusive prefix over reversed bins (first 4 waves)
    // (tid < 256 selects whole waves 0..3, so the shuffles stay wave-uniform)
    uint32_t c = 0, incl = 0;
    if (tid < 256) {
      c = sh.tot[255 - tid];
      incl = c;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      if (lane == 63) sh.wscan[w] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t base = 0;
      for (int i = 0; i < w; ++i) base += sh.wscan[i];
      incl += base;
      const uint32_t excl = incl - c;
      if (excl < krem && krem <= incl) {
        sh.digit = 255u - tid;
        sh.above = excl;
        sh.in_dig = c;
      }
    }
    __syncthreads();
    const uint32_t d = sh.digit;
    krem -= sh.above;
    eq_total = sh.in_dig;
    prefix |= d << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the key K of the budget-th largest score; krem (>= 1) cells
  // with key == K are taken, lowest index first; eq_total cells have key K.
  const uint32_t K = prefix;
  const bool all_eq = (eq_total == krem);
  uint32_t sel_base = 0, eq_base = 0;
  for (int64_t base = 0; base < n; base += kTopkThreads) {
    const int64_t i = base + tid;
    uint32_t key = 0;
    if (i < n) key = score_key(s[i]);
    const bool gt = (i < n) && key > K;
    const bool eq = (i < n) && key == K;
    bool sel;
    if (all_eq) {
      sel = gt || eq;
    } else {
      uint32_t eq_round = 0;
      const uint32_t eq_rank = eq_base + block_excl_scan(eq, sh.wscan, eq_round);
      eq_base += eq_round;
      sel = gt || (eq && eq_rank < krem);
    }
    uint32_t sel_round = 0;
    const uint32_t pos = sel_base + block_excl_scan(sel, sh.wscan2, sel_round);
    sel_base += sel_round;
    if (sel && pos < (uint32_t)budget) out[pos] = (int32_t)i;  // exactly budget by construction
  }
}

hipError_t launch_topk(const float* scores, int32_t* ids, int T, int pos0, int G, int budget,
                       int64_t n_cells, hipStream_t stream) {
  dim3 grid(T * G), block(kTopkThreads);
  topk_kernel<<<grid, block, 0, stream>>>(scores, ids, T, pos0, G, budget, n_cells);
  return hipGetLastError();
}

}  // namespace qsa
