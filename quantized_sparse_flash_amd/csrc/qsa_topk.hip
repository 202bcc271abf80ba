// qsa_topk.hip -- selected ids of every (token, group) row.
//
// Pages: "round 6 track b - qsa flash" (delivered change: identity ids when
// the token sees at most 2051 cells, explicit selection above that, also
// inside chunks that cross the threshold; experiment contract: the selected-
// index semantics above budget are kept).  Tie rule and order (lower index
// first on equal scores, ids ascending) are this library's reading.
//
// One workgroup per row.  Identity rows are written directly.  Above budget
// the row's scores become order-preserving 32-bit keys and an MSB-first
// radix select finds K, the key of the budget-th largest score, and krem,
// how many cells with key == K are taken (the lowest-index ones).  The
// selected cells are then every key > K plus those krem, written in
// ascending index order.
//
//   topk_regs_kernel (rows of at most 512 x 32 cells): the row is read from
//     HBM once, coalesced, into registers (EPT keys per thread).  A sample
//     of 1024 cells spread over the row gives a threshold that leaves, as a rule,
//     a few thousand keys at or above it; those are counted exactly and
//     copied to an LDS list, and three radix passes of 11, 11 and 10 bits
//     (LDS atomics) run over the list alone.  When the list would not hold
//     budget..6144 keys, the passes run over the registers instead (every
//     key in the first pass, then only keys that match the prefix found so
//     far).  Each pass's digit search zeroes the bins it reads, and its
//     scans alternate between two buffers, so a pass costs two barriers and
//     no separate clearing.  The selection is then two LDS bitmaps over
//     the row's cells (key > K, key == K), built from one ballot per 64
//     cells, and two block-wide scans over the bitmap words: the first keeps
//     the first krem equal keys, the second gives every selected cell its
//     output position.
//
//   topk_list_kernel (rows of 512 x 32 + 1 .. 512 x 64 cells): the same
//     select on a list of (key, cell) pairs that the row, streamed from
//     HBM, leaves at or above the sampled threshold (see there).
//
//   topk_stream_kernel (longer rows): the same radix select with 8-bit
//     digits, re-reading the row from memory in each of four passes, and an
//     ordered ballot compaction.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

// Order-preserving key: larger float -> larger unsigned; -0.0 == +0.0
// (x + 0 turns -0 into +0 under round-to-nearest; then negative values have
// all bits flipped, positive ones only the sign bit).  NaN inputs are
// unsupported; -inf maps to 0x007fffff, so key 0 is below every real score
// and marks cells outside the row.
__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP: shifts by 1, 2,
// 4 and 8 lanes inside each 16-lane row, then row_bcast:15 / row_bcast:31
// carry row totals into the rows above (gfx9-family DPP controls; lanes
// without a source add the 0 passed as `old`).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum of v over a block of NT threads in thread order;
// writes the block total.  `wsum` holds NT / 64 words; two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int w = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(v);
  if ((threadIdx.x & 63) == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t c = wsum[i];
    base += (i < w) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// The same with one barrier: the caller alternates between two `wsum`
// buffers, so a buffer is rewritten only two calls later, after the middle
// call's barrier has passed every read of it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_sum1(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int w = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(v);
  if ((threadIdx.x & 63) == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t c = wsum[i];
    base += (i < w) ? c : 0u;
    tot += c;
  }
  total = tot;
  return base + incl - v;
}

// Identity row: 0 .. n-1, then -1 padding.
__device__ __forceinline__ void write_identity(int32_t* out, int64_t n, int budget, int nt) {
  for (int i = threadIdx.x; i < budget; i += nt) out[i] = (i < n) ? i : -1;
}

// One radix step of the select: the 11-bit digit (at `shift`) of the
// krem-th largest key still in play, read from the 2048-bin histogram `h`
// (kCopies copies, 2048 words apart, added up), bins in key order; it is
// or-ed into `prefix`, krem drops by the keys of higher digits and eq_count
// is the count in the chosen bin.  Thread tid owns bins 2047 - 4 tid - q
// (q < 4: one 16-byte word, element 3 - q) and zeroes them, so the next
// histogram starts from zero after the barrier inside.  `parity` alternates
// the scan buffers (wsum: 2 x NT / 64 words) and result words (res: 3 x 2)
// between calls, so a call costs two barriers.
template <int NT, int kCopies>
__device__ __forceinline__ void choose_digit(uint32_t* h, int shift, uint32_t& prefix,
                                             uint32_t& krem, uint32_t& eq_count, int& parity,
                                             uint32_t* wsum, uint32_t* res) {
  static_assert(4 * NT == 2048, "four bins per thread");
  const int tid = threadIdx.x;
  const int b0 = 2044 - 4 * tid;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 v = *reinterpret_cast<const u32x4*>(&h[b0]);
  *reinterpret_cast<u32x4*>(&h[b0]) = zero;
#pragma unroll
  for (int cp = 1; cp < kCopies; ++cp) {
    v += *reinterpret_cast<const u32x4*>(&h[2048 * cp + b0]);
    *reinterpret_cast<u32x4*>(&h[2048 * cp + b0]) = zero;
  }
  uint32_t c[4], mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = v[3 - q];
    mine += c[q];
  }
  parity ^= 1;
  const int p = parity;
  uint32_t total;
  const uint32_t excl = block_excl_sum1<NT>(mine, wsum + p * (NT / 64), total);
  if (excl < krem && krem <= excl + mine) {  // exactly one thread
    uint32_t acc = excl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (acc < krem && krem <= acc + c[q]) {
        res[p] = 4u * tid + q;  // 2047 - digit
        res[2 + p] = acc;
        res[4 + p] = c[q];
      }
      acc += c[q];
    }
  }
  __syncthreads();
  prefix |= (2047u - res[p]) << shift;
  krem -= res[2 + p];
  eq_count = res[4 + p];
}

// The selection in ascending cell order from two bitmaps over the row's
// cells (bit c of word c / 32): bm_gt holds the selected cells when every
// key equal to K is taken (take_all_eq), else the cells with key > K, and
// bm_eq those with key == K, of which the first krem in index order are
// taken.  Thread tid owns words [kWpt tid, +kWpt); one block-wide scan keeps
// the first krem equal keys, a second gives every selected cell its output
// position.  Exactly `budget` ids are written.
template <int NT, int kWords>
__device__ __forceinline__ void write_selection(const uint32_t* bm_gt, const uint32_t* bm_eq,
                                                bool take_all_eq, uint32_t krem, int32_t* out,
                                                int budget, int& parity, uint32_t* wsum) {
  constexpr int kWpt = (kWords + NT - 1) / NT;  // words per thread
  const int tid = threadIdx.x;
  auto excl_sum = [&](uint32_t v, uint32_t& total) {
    parity ^= 1;
    return block_excl_sum1<NT>(v, wsum + parity * (NT / 64), total);
  };
  uint32_t sel[kWpt];
#pragma unroll
  for (int k = 0; k < kWpt; ++k) {
    const int wd = kWpt * tid + k;
    sel[k] = wd < kWords ? bm_gt[wd] : 0u;
  }
  if (!take_all_eq) {  // ties at K: only the first krem of them, in index order
    uint32_t n_eq = 0;
#pragma unroll
    for (int k = 0; k < kWpt; ++k) {
      const int wd = kWpt * tid + k;
      n_eq += wd < kWords ? __popc(bm_eq[wd]) : 0u;
    }
    uint32_t eq_total;
    uint32_t rank = excl_sum(n_eq, eq_total);
#pragma unroll
    for (int k = 0; k < kWpt; ++k) {
      const int wd = kWpt * tid + k;
      uint32_t e = wd < kWords ? bm_eq[wd] : 0u;
      while (e) {
        const uint32_t bit = e & (0u - e);
        if (rank < krem) sel[k] |= bit;
        ++rank;
        e ^= bit;
      }
    }
  }
  uint32_t n_sel = 0;
#pragma unroll
  for (int k = 0; k < kWpt; ++k) n_sel += __popc(sel[k]);
  uint32_t sel_total;
  uint32_t pos = excl_sum(n_sel, sel_total);  // sel_total == budget
#pragma unroll
  for (int k = 0; k < kWpt; ++k) {
    uint32_t b = sel[k];
    const int base = 32 * (kWpt * tid + k);
    while (b) {
      const int bit = __builtin_ctz(b);
      if (pos < (uint32_t)budget) out[pos] = base + bit;  // exactly budget by construction
      ++pos;
      b &= b - 1u;
    }
  }
}

}  // namespace

// ------------------------------------------------------------ register rows
constexpr int kRegThreads = 512;
constexpr int kListCap = 6144;    // survivors of the first digit kept in LDS

template <int EPT>
__global__ __launch_bounds__(kRegThreads) __attribute__((amdgpu_waves_per_eu(4))) void
topk_regs_kernel(const float* __restrict__ scores,
                                                                int32_t* __restrict__ ids, int G,
                                                                int pos0, int budget,
                                                                int64_t n_cells) {
  constexpr int NT = kRegThreads, NW = NT / 64;
  constexpr int kWords = NT * EPT / 32;         // bitmap words per row
  // hist[0] serves every pass; in the first pass hist[1..3] are extra copies
  // (one per 16-lane quarter of a wave, fewer same-bin atomic collisions),
  // afterwards their space holds the survivors of the first digit
  __shared__ __attribute__((aligned(16))) uint32_t hist[4][2048];
  uint32_t* const list = &hist[1][0];
  static_assert(3 * 2048 >= kListCap, "survivor list fits in hist[1..3]");
  __shared__ __attribute__((aligned(8))) uint32_t bm_gt[kWords], bm_eq[kWords];  // key > K (or >=), == K
  __shared__ uint32_t wsum[2][NW], wcount[NW];
  __shared__ uint32_t s_res[6];  // choose_digit's result words
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x;  // t * G + g
  const int64_t n = (int64_t)pos0 + row / G + 1;
  int32_t* out = ids + (int64_t)row * budget;
  if (n <= budget) {
    write_identity(out, n, budget, NT);
    return;
  }

  // ---- cell tid + NT i of the row -> key[i] (0 past the row's end).  Raw
  // buffer loads: slice i (cells NT i ..) gets a resource of its own, built
  // on the scalar unit, whose size stops at the row's end, so the hardware
  // range check returns 0 past it; every load is unconditional (all in
  // flight at once) and uses the one lane offset 4 tid.
  const int n32 = (int)n;  // <= NT * EPT
  const float* srow = scores + (int64_t)row * n_cells;
  uint32_t key[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int start = min(NT * i, n32);  // at most one past the row's end
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(srow + start), (short)0, 4 * (n32 - start), kBufferFlags);
    key[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * tid, 0, 0);
    // fence every 8 loads: the scheduler would otherwise hoist all EPT
    // resources (4 scalar registers each) ahead of the loads
    if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }

  // ---- radix select, most significant digit first.  The block finds the
  // digit of the krem-th largest remaining key from a histogram `h`.
  uint32_t prefix = 0, krem = (uint32_t)budget, eq_count = 0;
  int parity = 0;  // alternates the scan and result buffers between calls
  auto excl_sum = [&](uint32_t v, uint32_t& total) {
    parity ^= 1;
    return block_excl_sum1<NT>(v, &wsum[parity][0], total);
  };
  auto choose = [&](int shift, auto copies) {
    choose_digit<NT, decltype(copies)::value>(&hist[0][0], shift, prefix, krem, eq_count, parity,
                                              &wsum[0][0], s_res);
  };
  using One = std::integral_constant<int, 1>;
  using Four = std::integral_constant<int, 4>;
  auto clear_hist = [&](int words) {
    for (int b = tid; b < words; b += NT) (&hist[0][0])[b] = 0u;
    __syncthreads();
  };

  // every key, converted (cells past the row's end get key 0)
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    key[i] = score_key(__builtin_bit_cast(float, key[i]));
    if (NT * (i + 1) > n32)  // slice reaches past the row's end (a scalar test)
      key[i] = tid < n32 - NT * i ? key[i] : 0u;
  }

  // ---- a threshold from a sample.  Every thread contributes two of the
  // row's cells (below); the digit (bits 31..21) of the sample's r-th largest
  // key, r set four standard deviations above the sample's expected count
  // of selected cells, gives t = digit << 21, which usually leaves between
  // budget and kListCap keys at or above it.  Those keys go to the list and
  // the exact select runs on them alone (the budget-th largest key of the
  // row is the budget-th largest of the list whenever the list holds at
  // least budget keys).  Otherwise the full passes below run.  Rows of at
  // most 8 keys per thread (4,096 cells) skip the sample: there the full
  // passes are the shorter way (9.2 against 10.6 us for 16 rows of ~2,050
  // cells, 7.0 against 8.0 us for 2 rows of 4,001), while at 8,200 cells
  // they took 17.2 against 11.4 us.
  bool listed = false;
  if constexpr (EPT > 8) {
    // The sample comes from the registers: wave w's lanes take their keys
    // of slices i = s (EPT / 16) (mod EPT) for s = 2 w and 2 w + 1, i.e.
    // cells NT i + 64 w + lane: sixteen runs of 64 cells spread evenly over
    // the row (no cell twice).  Cells past the row's end hold key 0, below
    // every score, and are left out of the expected count.
    constexpr int kStride = EPT >= 16 ? EPT / 16 : 1;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // in a scalar register
    uint32_t smp[2] = {0u, 0u};
#pragma unroll
    for (int c = 0; c < NW; ++c)  // one case per wave: two selects each
      if (c == wu) {
        smp[0] = key[((2 * c) * kStride) % EPT];
        smp[1] = key[((2 * c + 1) * kStride) % EPT];
      }
    int n_smp = 0;  // sampled cells inside the row (the same in every thread)
#pragma unroll
    for (int ws = 0; ws < 2 * NW; ++ws)
      n_smp += min(max(n32 - (NT * (((ws * kStride) % EPT)) + 64 * (ws >> 1)), 0), 64);
    clear_hist(2048);
    atomicAdd(&hist[0][smp[0] >> 21], 1u);
    atomicAdd(&hist[0][smp[1] >> 21], 1u);
    __syncthreads();
    const float expect = (float)budget * (float)n_smp / (float)n32;
    const uint32_t r = (uint32_t)fminf(expect + 4.0f * sqrtf(expect) + 1.0f, (float)n_smp);
    krem = r;
    choose(21, One{});
    const uint32_t t = prefix;  // the sample digit, bits 20..0 zero
    prefix = 0;
    krem = (uint32_t)budget;
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) mine += key[i] >= t ? 1u : 0u;
    uint32_t n_at;
    uint32_t pos = excl_sum(mine, n_at);
    if (n_at >= (uint32_t)budget && n_at <= (uint32_t)kListCap) {
      listed = true;
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (key[i] >= t) list[pos++] = key[i];
      __syncthreads();  // publishes the list (hist[0] is zero: choose cleared it)
      for (int j = tid; j < (int)n_at; j += NT) atomicAdd(&hist[0][list[j] >> 21], 1u);
      __syncthreads();
      choose(21, One{});
      for (int j = tid; j < (int)n_at; j += NT) {
        const uint32_t k = list[j];
        if ((k >> 21) == (prefix >> 21)) atomicAdd(&hist[0][(k >> 10) & 0x7ffu], 1u);
      }
      __syncthreads();
      choose(10, One{});
      for (int j = tid; j < (int)n_at; j += NT) {
        const uint32_t k = list[j];
        if ((k >> 10) == (prefix >> 10)) atomicAdd(&hist[0][k & 0x3ffu], 1u);
      }
      __syncthreads();
      choose(0, One{});
    }
  }

  if (!listed) {
  // first digit: bits 31..21 of every key (fences every 8 keys keep the
  // scheduler from computing all bin addresses at once)
  clear_hist(4 * 2048);
  {
    uint32_t* h = hist[lane >> 4];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      atomicAdd(&h[key[i] >> 21], 1u);
      if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  choose(21, Four{});
  const uint32_t d1 = prefix >> 21;
  const uint32_t n1 = eq_count;  // keys whose first digit is d1 (they hold the answer)
  if (n1 <= (uint32_t)kListCap) {
    // survivors of the first digit -> list, wave by wave in cell order
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) cnt += __popcll(__ballot((key[i] >> 21) == d1));
    if (lane == 0) wcount[w] = cnt;
    __syncthreads();  // publishes wcount
    uint32_t pos = 0;
    for (int v = 0; v < w; ++v) pos += wcount[v];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const bool hit = (key[i] >> 21) == d1;
      const uint64_t m = __ballot(hit);
      if (hit) list[pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
          key[i];
      pos += __popcll(m);
    }
    __syncthreads();
    // second digit (bits 20..10) and third (bits 9..0) over the list
    for (int j = tid; j < (int)n1; j += NT) atomicAdd(&hist[0][(list[j] >> 10) & 0x7ffu], 1u);
    __syncthreads();
    choose(10, One{});
    for (int j = tid; j < (int)n1; j += NT) {
      const uint32_t k = list[j];
      if ((k >> 10) == (prefix >> 10)) atomicAdd(&hist[0][k & 0x3ffu], 1u);
    }
    __syncthreads();
    choose(0, One{});
  } else {
    // too many survivors for the list: the same two digits over the registers
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if ((key[i] >> 21) == d1) atomicAdd(&hist[0][(key[i] >> 10) & 0x7ffu], 1u);
    __syncthreads();
    choose(10, One{});
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if ((key[i] >> 10) == (prefix >> 10)) atomicAdd(&hist[0][key[i] & 0x3ffu], 1u);
    __syncthreads();
    choose(0, One{});
  }
  }  // !listed
  const uint32_t K = prefix;  // krem (1 <= krem <= eq_count) cells with key K are taken

  // ---- bitmaps: element row i of wave w covers cells [NT i + 64 w, +64)
  // and its ballot is one 64-bit bitmap entry, stored by lane 0.  When every
  // cell with key K is taken (the usual case) one bitmap of key >= K is the
  // selection; otherwise key > K and key == K apart.
  const bool take_all_eq = eq_count == krem;
  uint64_t* const gt64 = reinterpret_cast<uint64_t*>(bm_gt);
  uint64_t* const eq64 = reinterpret_cast<uint64_t*>(bm_eq);
  if (take_all_eq) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const uint64_t g = __ballot(key[i] >= K);
      if (lane == 0) gt64[(NT * i + 64 * w) >> 6] = g;
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const uint64_t g = __ballot(key[i] > K);
      const uint64_t e = __ballot(key[i] == K);
      if (lane == 0) {
        gt64[(NT * i + 64 * w) >> 6] = g;
        eq64[(NT * i + 64 * w) >> 6] = e;
      }
    }
  }
  __syncthreads();

  write_selection<NT, kWords>(bm_gt, bm_eq, take_all_eq, krem, out, budget, parity, &wsum[0][0]);
}

// ------------------------------------------------------------ listed rows
// Rows of 16,385..32,768 cells (EPT = 64 slices of 512 cells).  The same
// select as topk_regs_kernel, but the row is streamed from HBM in batches of
// 16 slices and never held whole: after a sampled threshold t (here the top
// 22 bits of the sample's r-th largest key) only the cells with key >= t
// stay, as (key, cell) pairs in an LDS list (each wave reserves its batch's
// entries with one LDS atomic), and both the radix passes and the selection
// bitmaps (LDS atomic ors) work from the list.  Few registers and ~36 KB of
// LDS let four rows share a CU where the register kernel (64 keys per
// thread, 128 VGPRs) fits two: each row spends much of its time in barriers
// and LDS round trips, and the other rows' streaming fills those gaps.  A
// list that would overflow, or hold fewer than budget keys, sends the row
// to three radix passes and a bitmap pass that re-read it from memory.
constexpr int kListThreads = 512;
constexpr int kListEpt = 64;     // slices: rows up to 32,768 cells
constexpr int kListBatch = 16;   // slices in flight per thread
constexpr int kListPairs = 4608; // (key, cell) pairs the list holds
constexpr int kCachePolicyNt = 2;  // buffer-load cache policy: non-temporal (nt)

template <int EPT>
__global__ __launch_bounds__(kListThreads) __attribute__((amdgpu_waves_per_eu(8))) void
topk_list_kernel(const float* __restrict__ scores, int32_t* __restrict__ ids, int G, int pos0,
                 int budget, int64_t n_cells) {
  constexpr int NT = kListThreads, NW = NT / 64;
  constexpr int kWords = NT * EPT / 32;  // bitmap words per row
  static_assert(EPT % kListBatch == 0 && NT * EPT <= 65536, "cells fit 16 bits");
  // the two selection bitmaps reuse the histogram's words: the last digit
  // choice leaves every bin zero
  __shared__ __attribute__((aligned(16))) uint32_t hist[2048];
  static_assert(2 * kWords <= 2048, "bitmaps fit the histogram");
  uint32_t* const bm_gt = hist;
  uint32_t* const bm_eq = hist + kWords;
  __shared__ uint32_t lkey[kListPairs];
  __shared__ uint16_t lcell[kListPairs];
  __shared__ uint32_t wsum[2][NW];
  __shared__ uint32_t s_res[6];  // choose_digit's result words
  __shared__ uint32_t s_n;       // pairs reserved in the list
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x;  // t * G + g
  const int64_t n = (int64_t)pos0 + row / G + 1;
  int32_t* out = ids + (int64_t)row * budget;
  if (n <= budget) {
    write_identity(out, n, budget, NT);
    return;
  }
  const int n32 = (int)n;  // <= NT * EPT
  const float* srow = scores + (int64_t)row * n_cells;
  // cell NT i + tid (slice i): a raw buffer load whose resource stops at the
  // row's end, so the hardware range check returns 0 past it
  auto load_slice = [&](int i) -> uint32_t {
    const int start = min(NT * i, n32);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(srow + start), (short)0, 4 * (n32 - start), kBufferFlags);
    return __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * tid, 0, 0);
  };
  // the same load, non-temporal (cache policy nt), for the stream: each
  // score is read once there, and 0.5 GB of them no longer sweep the KV
  // cells that the attention launch after the top-k gathers out of the
  // Infinity Cache (long-context step 0.420 against 0.421 ms back to back,
  // single steps after a cache flush 0.455-0.481 against 0.499-0.509 ms).
  // The sample keeps the ordinary load: the stream reads those cells again
  // and finds them in L2.
  auto load_slice_nt = [&](int i) -> uint32_t {
    const int start = min(NT * i, n32);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(srow + start), (short)0, 4 * (n32 - start), kBufferFlags);
    return __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * tid, 0, kCachePolicyNt);
  };
  // its key, 0 past the row's end (below every score)
  auto key_of = [&](uint32_t bits, int i) -> uint32_t {
    const uint32_t k = score_key(__builtin_bit_cast(float, bits));
    return NT * i + tid < n32 ? k : 0u;
  };

  uint32_t prefix = 0, krem = (uint32_t)budget, eq_count = 0;
  int parity = 0;
  auto choose = [&](int shift) {
    choose_digit<NT, 1>(hist, shift, prefix, krem, eq_count, parity, &wsum[0][0], s_res);
  };

  // ---- the sample: as in topk_regs_kernel, wave w takes slices
  // s (EPT / 16) for s = 2 w, 2 w + 1 (cells NT i + tid): sixteen runs of
  // 64 cells spread evenly over the row.  Histogram and bitmaps are cleared
  // while those loads are in flight.
  constexpr int kStride = EPT / 16;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int is0 = (2 * wu) * kStride, is1 = (2 * wu + 1) * kStride;
  const uint32_t smp_bits0 = load_slice(is0), smp_bits1 = load_slice(is1);
  // the first batch of the stream below is requested now: it arrives while
  // the sample picks the threshold
  uint32_t k[kListBatch];
#pragma unroll
  for (int j = 0; j < kListBatch; ++j) k[j] = load_slice_nt(j);
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&hist[4 * tid]) = zero;
    if (tid == 0) s_n = 0;
  }
  int n_smp = 0;  // sampled cells inside the row (the same in every thread)
#pragma unroll
  for (int ws = 0; ws < 2 * NW; ++ws)
    n_smp += min(max(n32 - (NT * ws * kStride + 64 * (ws >> 1)), 0), 64);
  __syncthreads();
  atomicAdd(&hist[key_of(smp_bits0, is0) >> 21], 1u);
  atomicAdd(&hist[key_of(smp_bits1, is1) >> 21], 1u);
  __syncthreads();
  {
    const float expect = (float)budget * (float)n_smp / (float)n32;
    krem = (uint32_t)fminf(expect + 4.0f * sqrtf(expect) + 1.0f, (float)n_smp);
  }
  choose(21);
  // and the next 11 bits among the samples of that digit: t is the top 22
  // bits of the sample's r-th largest key, which leaves fewer extra cells in
  // the list than the digit alone (the cells of its 11-bit bin)
  {
    const uint32_t k0 = key_of(smp_bits0, is0), k1 = key_of(smp_bits1, is1);
    if ((k0 >> 21) == (prefix >> 21)) atomicAdd(&hist[(k0 >> 10) & 0x7ffu], 1u);
    if ((k1 >> 21) == (prefix >> 21)) atomicAdd(&hist[(k1 >> 10) & 0x7ffu], 1u);
  }
  __syncthreads();
  choose(10);
  const uint32_t t = prefix;  // bits 9..0 zero
  prefix = 0;
  krem = (uint32_t)budget;

  // ---- stream the row: keys >= t join the list.  Per batch, each wave
  // places its hits by ballots (slice by slice, in lane order) and reserves
  // them with one LDS atomic; pairs past the list's end are dropped and the
  // count tells that it overflowed.
  for (int b = 0; b < EPT; b += kListBatch) {
    if (b > 0) {
#pragma unroll
      for (int j = 0; j < kListBatch; ++j) k[j] = load_slice_nt(b + j);
    }
    uint32_t off[kListBatch];  // hits of the wave's earlier slices, plus the lane's rank
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < kListBatch; ++j) {
      k[j] = key_of(k[j], b + j);
      const uint64_t m = __ballot(k[j] >= t);
      off[j] = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      run += (uint32_t)__popcll(m);
    }
    uint32_t base = 0;
    if (lane == 0 && run) base = atomicAdd(&s_n, run);
    base = __builtin_amdgcn_readlane(base, 0);
#pragma unroll
    for (int j = 0; j < kListBatch; ++j) {
      const uint32_t pos = base + off[j];
      if (k[j] >= t && pos < (uint32_t)kListPairs) {
        lkey[pos] = k[j];
        lcell[pos] = (uint16_t)(NT * (b + j) + tid);
      }
    }
  }
  __syncthreads();
  const uint32_t n_at = s_n;
  const bool listed = n_at >= (uint32_t)budget && n_at <= (uint32_t)kListPairs;

  if (listed) {
    // ---- exact select over the list: digits 31..21, 20..10, 9..0
    for (int j = tid; j < (int)n_at; j += NT) atomicAdd(&hist[lkey[j] >> 21], 1u);
    __syncthreads();
    choose(21);
    for (int j = tid; j < (int)n_at; j += NT) {
      const uint32_t kj = lkey[j];
      if ((kj >> 21) == (prefix >> 21)) atomicAdd(&hist[(kj >> 10) & 0x7ffu], 1u);
    }
    __syncthreads();
    choose(10);
    for (int j = tid; j < (int)n_at; j += NT) {
      const uint32_t kj = lkey[j];
      if ((kj >> 10) == (prefix >> 10)) atomicAdd(&hist[kj & 0x3ffu], 1u);
    }
    __syncthreads();
    choose(0);
  } else {
    // ---- the same three digits over the row, re-read from memory
    for (int b = 0; b < EPT; ++b) atomicAdd(&hist[key_of(load_slice(b), b) >> 21], 1u);
    __syncthreads();
    choose(21);
    for (int b = 0; b < EPT; ++b) {
      const uint32_t kb = key_of(load_slice(b), b);
      if ((kb >> 21) == (prefix >> 21)) atomicAdd(&hist[(kb >> 10) & 0x7ffu], 1u);
    }
    __syncthreads();
    choose(10);
    for (int b = 0; b < EPT; ++b) {
      const uint32_t kb = key_of(load_slice(b), b);
      if ((kb >> 10) == (prefix >> 10)) atomicAdd(&hist[kb & 0x3ffu], 1u);
    }
    __syncthreads();
    choose(0);
  }
  const uint32_t K = prefix;  // krem (1 <= krem <= eq_count) cells with key K are taken
  const bool take_all_eq = eq_count == krem;

  // ---- bitmaps (zero: see above): every cell with key >= K is in the list
  // when it is used (K >= t), so its pairs set the bits; otherwise one more
  // pass over the row, a ballot per 64 cells
  if (listed) {
    for (int j = tid; j < (int)n_at; j += NT) {
      const uint32_t kj = lkey[j];
      const uint32_t c = lcell[j];
      const uint32_t bit = 1u << (c & 31u);
      if (take_all_eq ? kj >= K : kj > K)
        atomicOr(&bm_gt[c >> 5], bit);
      else if (!take_all_eq && kj == K)
        atomicOr(&bm_eq[c >> 5], bit);
    }
  } else {
    uint64_t* const gt64 = reinterpret_cast<uint64_t*>(bm_gt);
    uint64_t* const eq64 = reinterpret_cast<uint64_t*>(bm_eq);
    for (int b = 0; b < EPT; ++b) {
      const uint32_t kb = key_of(load_slice(b), b);
      const uint64_t g = __ballot(take_all_eq ? kb >= K : kb > K);
      const uint64_t e = __ballot(kb == K);
      if (lane == 0) {
        gt64[(NT * b + 64 * w) >> 6] = g;
        if (!take_all_eq) eq64[(NT * b + 64 * w) >> 6] = e;
      }
    }
  }
  __syncthreads();
  write_selection<NT, kWords>(bm_gt, bm_eq, take_all_eq, krem, out, budget, parity, &wsum[0][0]);
}

// ------------------------------------------------------------- streamed rows
constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / 64;

__global__ __launch_bounds__(kStreamThreads) void topk_stream_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ ids, int G, int pos0, int budget,
    int64_t n_cells) {
  __shared__ uint32_t hist[kStreamWaves][256];
  __shared__ uint32_t wsum[kStreamWaves];
  __shared__ uint32_t s_digit, s_above, s_count;
  const int row = blockIdx.x;
  const int64_t n = (int64_t)pos0 + row / G + 1;
  int32_t* out = ids + (int64_t)row * budget;
  const int tid = threadIdx.x, w = tid >> 6;
  if (n <= budget) {
    write_identity(out, n, budget, kStreamThreads);
    return;
  }
  const float* s = scores + (int64_t)row * n_cells;

  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)budget, eq_count = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kStreamWaves * 256; i += kStreamThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kStreamThreads) {
      const uint32_t key = score_key(s[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t c = 0;
    if (tid < 256) {
#pragma unroll
      for (int i = 0; i < kStreamWaves; ++i) c += hist[i][255 - tid];  // descending digits
    }
    uint32_t total;
    const uint32_t excl = block_excl_sum<kStreamThreads>(tid < 256 ? c : 0u, wsum, total);
    if (tid < 256 && excl < krem && krem <= excl + c) {
      s_digit = 255u - tid;
      s_above = excl;
      s_count = c;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    krem -= s_above;
    eq_count = s_count;
    __syncthreads();
  }
  const uint32_t K = prefix;
  const bool all_eq = eq_count == krem;
  uint32_t sel_base = 0, eq_base = 0;
  for (int64_t base = 0; base < n; base += kStreamThreads) {
    const int64_t i = base + tid;
    const uint32_t key = i < n ? score_key(s[i]) : 0u;
    const bool gt = i < n && key > K;
    const bool eq = i < n && key == K;
    bool sel = gt || (all_eq && eq);
    if (!all_eq) {
      uint32_t eq_round;
      const uint32_t eq_rank = eq_base + block_excl_sum<kStreamThreads>(eq, wsum, eq_round);
      eq_base += eq_round;
      sel = gt || (eq && eq_rank < krem);
    }
    uint32_t sel_round;
    const uint32_t pos = sel_base + block_excl_sum<kStreamThreads>(sel, wsum, sel_round);
    sel_base += sel_round;
    if (sel && pos < (uint32_t)budget) out[pos] = (int32_t)i;  // exactly budget by construction
  }
}

hipError_t launch_topk(const float* scores, int32_t* ids, int T, int pos0, int G, int budget,
                       int64_t n_cells, hipStream_t stream) {
  const dim3 grid(T * G);
  const int64_t n_max = (int64_t)pos0 + T;  // longest row
  const int64_t per = (n_max + kRegThreads - 1) / kRegThreads;
  if (per <= 8) {
    topk_regs_kernel<8><<<grid, kRegThreads, 0, stream>>>(scores, ids, G, pos0, budget, n_cells);
  } else if (per <= 16) {
    topk_regs_kernel<16><<<grid, kRegThreads, 0, stream>>>(scores, ids, G, pos0, budget, n_cells);
  } else if (per <= 32) {
    topk_regs_kernel<32><<<grid, kRegThreads, 0, stream>>>(scores, ids, G, pos0, budget, n_cells);
  } else if (per <= kListEpt) {
    topk_list_kernel<kListEpt>
        <<<grid, kListThreads, 0, stream>>>(scores, ids, G, pos0, budget, n_cells);
  } else {
    topk_stream_kernel<<<grid, kStreamThreads, 0, stream>>>(scores, ids, G, pos0, budget,
                                                           n_cells);
  }
  return hipGetLastError();
}

}  // namespace qsa
