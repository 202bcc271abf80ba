// qsa_flash_rows.hip -- attention over one (token, group) row per wavefront.
//
// Pages: "opus_r9_qsa" (what changed: per 64-cell chunk, S for the group's
// 12 heads is combined and multiplied by 1/16, the softmax keeps a running
// max and sum, P is formed in fp16 and accumulated against V) and "round 6
// track b - qsa flash" (delivered change: identity ids derived in the kernel
// when the token sees at most `budget` cells, explicit ids above; scales are
// staged once per selected cell).  Split mode writes the per-chunk (o, m, l)
// records that "round 27 track b - qsa prep and merge" merges.
//
// Two kernels.  flash_split_kernel computes one 64-cell chunk of one
// (token, group) row per wavefront and writes its (o, m, l) record (split
// mode, the decode path).  flash_rows_staged_kernel (further down) attends a
// whole row per wavefront, its gathers staged through LDS one stage ahead
// (prompt tokens above budget), or, in its pieces form, a run of a row's
// chunks per wavefront with one record per piece (calls with few rows, whose
// rows alone would leave most SIMDs idle).  Work mapping of the split kernel
// (gfx950, wave64), shared in its PV half by the staged kernel:
//   * lane l: n = l % 16 is a query column (head n of the group, n < 12;
//     columns 12..15 carry zero queries), j = l / 16 a k-slot group;
//   * S^T[64 cells][16 queries] = K Q^T on v_mfma_f32_16x16x32_f16: A = K
//     (row = cell), B = Q^T, k = head dim.  Dim d of k-step s, slot (j, i)
//     is 64*(s/2) + 16*j + 8*(s%2) + i, so one 16-byte load per scale block
//     feeds two k-steps and each lane's codes share one K scale;
//   * the softmax runs on the S^T accumulators: every lane holds one query
//     and 16 cells, so row max/sum need only two cross-lane steps;
//   * O^T[256 dims][16 queries] += V^T P^T: B = P^T comes straight from the
//     S^T registers (the accumulator layout of two 16-cell tiles is exactly
//     the B layout of one 32-cell k-step); A = V^T uses dim d = 16*r + mt for
//     row r of m-tile mt, so a lane reads 16 contiguous codes of each of its
//     8 cells once and byte-selects them for all 16 m-tiles;
//   * int8 -> fp16 is one SDWA convert per element, then a packed fp16
//     multiply by the cell's scale (k and v rounded to fp16 once).
#include <type_traits>
#include <utility>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

constexpr float kLazyGrowth = 8.0f;  // log2 headroom of the running reference max
constexpr int kXcds = 8;             // XCDs that workgroups are dealt to, round robin


__device__ __forceinline__ half2_t splat_lo(uint32_t u) {
  const half2_t h = as_h2(u);
  return half2_t{h[0], h[0]};
}
__device__ __forceinline__ half2_t splat_hi(uint32_t u) {
  const half2_t h = as_h2(u);
  return half2_t{h[1], h[1]};
}


// One wave per (token, group, chunk) item.  Two waves per SIMD (at most 256
// registers each): the gathers are latency-bound, and the second wave's
// loads overlap the first one's arithmetic.  K and V go out together (one
// memory round trip).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void flash_split_kernel(RowArgs a) {
  const int lane = threadIdx.x & 63;
  const int G = a.G, H = G * kHpg;
  // wave-uniform: every per-row value below lives in scalar registers
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (item >= a.n_items) return;
  const int g = item % G;
  const int k = (item / G) % a.KC;
  const int t = item / (G * a.KC);
  const int64_t nkv = (int64_t)a.pos0 + t + 1;
  const bool explicit_ids = nkv > a.budget;
  const int nsel = explicit_ids ? a.budget : (int)nkv;
  const int nch = (nsel + kChunk - 1) / kChunk;
  if (k >= nch) return;

  const int n = lane & 15, j = lane >> 4;
  const bool qvalid = n < kHpg;
  const int hq = g * kHpg + (qvalid ? n : 0);

  // Q^T fragments (B operand of the score MFMA)
  half8_t qf[8];
  {
    const _Float16* qrow = a.q + ((int64_t)t * H + hq) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int d0 = 64 * (s >> 1) + 16 * j + 8 * (s & 1);
      qf[s] = qvalid ? *reinterpret_cast<const half8_t*>(qrow + d0) : half8_t{};
    }
  }

  const int8_t* kq_g = a.kq + (int64_t)g * a.n_cells * kHeadDim;
  const int8_t* vq_g = a.vq + (int64_t)g * a.n_cells * kHeadDim;
  const _Float16* ksc_g = a.ksc + (int64_t)g * a.n_cells * kNBlk;
  const _Float16* vsc_g = a.vsc + (int64_t)g * a.n_cells * kNBlk;

  // cell of chunk position `lane` (0 past the row), clamped into the cache
  const int cbase = k * kChunk;
  int my_cell;
  {
    const int p = cbase + lane;
    int c = p < nsel ? p : 0;
    if (explicit_ids) c = p < nsel ? a.ids[((int64_t)t * G + g) * a.budget + p] : 0;
    c = c < 0 ? 0 : c;
    my_cell = (int64_t)c >= a.n_cells ? (int)(a.n_cells - 1) : c;
  }

  // V codes and scales of k-step kk: lane (n, j) takes dims 16n..16n+15 of
  // the cells at positions 4j + i and 16 + 4j + i of the 32-cell half
  u32x4 vrow[2][8];
  uint32_t vs[2][8];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pos = 32 * kk + ((i < 4) ? (4 * j + i) : (16 + 4 * j + (i - 4)));
      const int cell = __shfl(my_cell, pos);
      vrow[kk][i] = *reinterpret_cast<const u32x4*>(vq_g + (int64_t)cell * kHeadDim + 16 * n);
      vs[kk][i] = *reinterpret_cast<const uint16_t*>(vsc_g + (int64_t)cell * kNBlk + (n >> 2));
    }

  // ---- S^T = K Q^T, four 16-cell m-tiles
  f32x4 sacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int cell = __shfl(my_cell, 16 * mt + n);
    const int8_t* krow = kq_g + (int64_t)cell * kHeadDim + 16 * j;
    const u32x2 ks = *reinterpret_cast<const u32x2*>(ksc_g + (int64_t)cell * kNBlk);
    u32x4 raw[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) raw[b] = *reinterpret_cast<const u32x4*>(krow + 64 * b);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const half2_t sc = (b == 0) ? splat_lo(ks.x) : (b == 1) ? splat_hi(ks.x)
                       : (b == 2) ? splat_lo(ks.y) : splat_hi(ks.y);
      uint32_t w[8];
      dq4(raw[b].x, sc, w[0], w[1]);
      dq4(raw[b].y, sc, w[2], w[3]);
      dq4(raw[b].z, sc, w[4], w[5]);
      dq4(raw[b].w, sc, w[6], w[7]);
      const half8_t a0 = __builtin_bit_cast(half8_t, u32x4{w[0], w[1], w[2], w[3]});
      const half8_t a1 = __builtin_bit_cast(half8_t, u32x4{w[4], w[5], w[6], w[7]});
      acc = mfma16(a0, qf[2 * b], acc);
      acc = mfma16(a1, qf[2 * b + 1], acc);
    }
    sacc[mt] = acc;
  }

  // ---- softmax over the chunk (base 2), relative to the chunk's own max
  float x[4][4];
  float cmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = cbase + 16 * mt + 4 * j + r;
      x[mt][r] = (p < nsel) ? sacc[mt][r] * kScoreScaleLog2 : -INFINITY;
      cmax = fmaxf(cmax, x[mt][r]);
    }
  cmax = wave_max_xor16_32(cmax);
  float lsum = 0.f;
  half8_t pb[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = fast_exp2(x[2 * kk + (i >> 2)][i & 3] - cmax);
      lsum += p;
      pb[kk][i] = (_Float16)p;
    }
  }
  const float l_chunk = wave_sum_xor16_32(lsum);

  // ---- O^T = V^T P^T, two 32-cell k-steps, 16 dim m-tiles
  f32x4 oacc[16];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    half2_t sp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[i] = as_h2(vs[kk][2 * i] | (vs[kk][2 * i + 1] << 16));
    static_for<16>([&](auto MT) {
      constexpr int mt = decltype(MT)::value;
      constexpr int dw = mt >> 2, by = mt & 3;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = as_u32(col_pair<by>(vrow[kk][2 * i][dw], vrow[kk][2 * i + 1][dw]) * sp[i]);
      const half8_t av = __builtin_bit_cast(half8_t, u32x4{w[0], w[1], w[2], w[3]});
      oacc[mt] = mfma16(av, pb[kk], oacc[mt]);
    });
  }

  if (!qvalid) return;
  float* rec = a.part + (((int64_t)t * a.KC + k) * H + hq) * kRec;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int mt = 0; mt < 16; mt += 2) {
      const float2 v = {oacc[mt][r], oacc[mt + 1][r]};
      *reinterpret_cast<float2*>(rec + 64 * j + 16 * r + mt) = v;
    }
  }
  if (j == 0) *reinterpret_cast<float2*>(rec + kHeadDim) = float2{cmax * kLn2, l_chunk};
}

// ------------------------------------------------------------------------
// Fused rows, staged through LDS.  The per-row attention of the split
// kernel (its PV half unchanged), in 32-cell stages whose gathers run one
// stage ahead of the math: K (codes and scales) of stage s + 1 is copied
// into the wave's LDS image as soon as K of stage s has been read out of it
// into registers, and V of stage s + 1 as soon as V of stage s has.  The
// copies are global_load_lds gathers (16 or 4 bytes per lane, no registers
// held); the ids of a chunk arrive the same way, two stages before its
// first copies are formed.  No other global load is in flight in the loop,
// so every wait names its count: at the top of stage s only V of stage s
// (9 copies) and, after an even stage, the ids copy before it may still be
// outstanding behind K of stage s; before the V phase only the 9 copies of
// the next K.  Two waves per SIMD cover each other's waits.
//
// S^T = K Q^T runs on the int8 MFMA: the K codes are its A operand as
// stored, Q is split once per row into two int8 pieces (q = sq (h + l/256),
// sq = max|q| / 127 over the row), every 64-dim block gives the exact
// integer products 256 I_hi + I_lo, and the cell's K scale of that block
// multiplies them in fp32.  The scores are exact in K and within sq / 512
// per element in Q (sq / 256 where the low piece saturates at 127), tighter
// than rounding each k = code * scale to fp16.
// PV keeps the fp16 MFMA with P rounded to fp16.
//
// Image of a wave (17,152 bytes): K codes | K scales | V codes | V scales |
// ids.  Cell c of a stage sits in code row r(c) = c ^ ((c >> 2) & 1) (an
// involution), and 16-byte piece p of a row at slot p ^ (row & 15); with
// these the K reads (16 cells, one piece each) and the V reads (one cell,
// 16 pieces, cells 4 j + i of the four lane groups) are free of bank
// conflicts whether the LDS serves 16 or 32 lanes of a 16-byte read per
// cycle.  Scales are in cell order (8 bytes per cell).
constexpr int kStage = 32;                        // cells per stage
constexpr int kStageCodes = kStage * kHeadDim;    // bytes of K (or V) codes
constexpr int kStageScales = kStage * kNBlk * 2;  // bytes of K (or V) scales
constexpr int kImgK = 0;
constexpr int kImgKs = kImgK + kStageCodes;
constexpr int kImgV = kImgKs + kStageScales;
constexpr int kImgVs = kImgV + kStageCodes;
constexpr int kImgIds = kImgVs + kStageScales;
constexpr int kImgBytes = kImgIds + 4 * kChunk;
constexpr int kCopiesPerHalf = kStage / 4 + 1;  // copies of K (or V) per stage

typedef __attribute__((address_space(3))) void* rows_lds_ptr_t;
__device__ __forceinline__ uint32_t rows_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(rows_lds_ptr_t)p;
}
__device__ __forceinline__ int stage_row(int c) { return c ^ ((c >> 2) & 1); }

// Copies from global memory straight into LDS: lane i's bytes land at LDS
// byte lds + size * i (lds wave-uniform, loaded into M0 by the asm).  Inline
// asm, so the compiler neither tracks them nor makes LDS reads wait for
// them; completion is awaited with the explicit vmcnt waits below.  The
// narrow forms take a 32-bit offset from a wave-uniform base, the wide
// forms a 64-bit address per lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_wide(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(addr), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_wide(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(addr), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
// Wait until at most 10, 9 or 0 of this wave's copies are outstanding; then
// until its LDS reads have returned.  The "memory" clobbers keep the
// compiler from moving LDS reads across them.
__device__ __forceinline__ void wait_copies_10() { asm volatile("s_waitcnt vmcnt(10)" : : : "memory"); }
__device__ __forceinline__ void wait_copies_9() { asm volatile("s_waitcnt vmcnt(9)" : : : "memory"); }
__device__ __forceinline__ void wait_copies_0() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }
#pragma clang diagnostic pop
static_assert(kCopiesPerHalf == 9, "the waits count 9 copies per K or V half");
__device__ __forceinline__ void wait_lds_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // the same wait, seen by the compiler
}

// PIECES: each wavefront attends one piece of a row, a.cpr consecutive
// 64-cell chunks of its selection (piece p: chunks a.cpr p ..), and writes
// the piece's (o, m, l) record for the merge instead of the row's output;
// a row under budget then takes its cells by position.
template <bool WIDE, bool PIECES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void flash_rows_staged_kernel(RowArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t img_all[4][kImgBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = a.G, H = G * kHpg;
  const int kcr = (a.KC + a.cpr - 1) / a.cpr;  // records per row (PIECES)
  int t, g, piece = 0;
  if constexpr (PIECES) {
    // (token, group, piece) per wavefront, a row's pieces consecutive
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
    if (item >= a.n_items) return;
    piece = item % kcr;
    g = (item / kcr) % G;
    t = item / (kcr * G);
  } else if (kXcds % G == 0) {
    // workgroups are dealt to the XCDs round robin: XCD x serves group
    // x % G only, so each XCD's L2 caches one group's cells
    const int per = kXcds / G;
    const int b = blockIdx.x, x = b % kXcds;
    const int r = __builtin_amdgcn_readfirstlane(4 * ((b / kXcds) * per + x / G) + wave);
    g = x % G;
    if (r >= a.n_items / G) return;
    t = a.T - 1 - r;  // longest rows first
  } else {
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
    if (item >= a.n_items) return;
    g = item % G;
    t = a.T - 1 - item / G;
  }
  uint8_t* img = img_all[wave];
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(rows_lds_addr(img));  // wave-uniform

  // Without PIECES only rows above budget come here (the tile kernel attends
  // the rest): every row selects exactly `budget` cells through its ids.  A
  // piece's row may be under budget (identity: cell = position); its ids
  // are then never read, and the ids copies, which keep the copy counts of
  // the waits below, read the launch's last row instead (above budget).
  const int64_t nkv = (int64_t)a.pos0 + t + 1;
  const bool identity = PIECES && nkv <= a.budget;
  const int nsel = identity ? (int)nkv : a.budget;
  const int nst = (nsel + kStage - 1) / kStage;
  int k_begin = 0, s_end = nst;  // this wavefront's chunks and stages
  if constexpr (PIECES) {
    const int nch = (nsel + kChunk - 1) / kChunk;
    k_begin = piece * a.cpr;
    if (k_begin >= nch) return;
    s_end = min(2 * min(k_begin + a.cpr, nch), nst);
  }
  const int s_begin = 2 * k_begin;

  const int n = lane & 15, j = lane >> 4;
  const bool qvalid = n < kHpg;
  const int hq = g * kHpg + (qvalid ? n : 0);

  // Q^T as the B operand of the int8 score MFMA.  Lane (n, j) holds dims
  // 64 b + 16 j + e (e < 16) of query n in byte e of qh[b] and ql[b]: the
  // positions at which it holds the same dims of the K codes.
  i32x4 qh[4], ql[4];
  float xs;  // log2-domain score per unit of K scale x (256 I_hi + I_lo)
  {
    const _Float16* qrow = a.q + ((int64_t)t * H + hq) * kHeadDim;
    half8_t qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int d0 = 64 * (s >> 1) + 16 * j + 8 * (s & 1);
      qf[s] = qvalid ? *reinterpret_cast<const half8_t*>(qrow + d0) : half8_t{};
    }
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)qf[s][i]));
    amax = wave_max_xor16_32(amax);
    const float inv = amax > 0.f ? 127.f / amax : 0.f;
    xs = (amax / 127.f) * (kScoreScaleLog2 / 256.f);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t hw = 0, lw = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * w + e;  // dim 64 b + 16 j + idx
          const float u = (float)qf[2 * b + (idx >> 3)][idx & 7] * inv;
          const float h = rintf(u);
          const float l = fminf(fmaxf(rintf((u - h) * 256.f), -127.f), 127.f);
          hw |= ((uint32_t)(int)h & 0xFFu) << (8 * e);
          lw |= ((uint32_t)(int)l & 0xFFu) << (8 * e);
        }
        qh[b][w] = (int)hw;
        ql[b][w] = (int)lw;
      }
    }
  }

  const int8_t* kq_g = a.kq + (int64_t)g * a.n_cells * kHeadDim;
  const int8_t* vq_g = a.vq + (int64_t)g * a.n_cells * kHeadDim;
  const _Float16* ksc_g = a.ksc + (int64_t)g * a.n_cells * kNBlk;
  const _Float16* vsc_g = a.vsc + (int64_t)g * a.n_cells * kNBlk;
  const int32_t* ids_row = a.ids + ((int64_t)(identity ? a.T - 1 : t) * G + g) * a.budget;
  auto clamp_cell = [&](int c) -> int {
    c = c < 0 ? 0 : c;
    return (int64_t)c >= a.n_cells ? (int)(a.n_cells - 1) : c;
  };

  // per-lane offsets of a stage's copies, shared by its K and V halves:
  // eight 16-byte code pieces (row 4 i + lane / 16, slot lane % 16) and one
  // scale dword (cell lane / 2, half lane % 2).  ids holds the cells of the
  // stage's chunk (lane = chunk position).
  // The cells are gathered by cross-lane shuffles well before the copies
  // (cells_of), the offsets formed from them only when the copies are due
  // (offsets_of), so no copy waits for a shuffle.
  using Off = typename std::conditional<WIDE, int64_t, uint32_t>::type;
  auto cells_of = [&](int s, int ids, int (&c)[kCopiesPerHalf]) {
    const int h = s & 1;
#pragma unroll
    for (int i = 0; i < kStage / 4; ++i)
      c[i] = __shfl(ids, kStage * h + stage_row(4 * i + (lane >> 4)));
    c[kStage / 4] = __shfl(ids, kStage * h + (lane >> 1));
  };
  auto offsets_of = [&](const int (&c)[kCopiesPerHalf], Off (&o)[kCopiesPerHalf]) {
#pragma unroll
    for (int i = 0; i < kStage / 4; ++i) {
      const int row = 4 * i + (lane >> 4);
      const int piece = (lane & 15) ^ (row & 15);
      o[i] = (Off)c[i] * kHeadDim + 16 * piece;
    }
    o[kStage / 4] = (Off)c[kStage / 4] * (2 * kNBlk) + 4 * (lane & 1);
  };
  auto issue_half = [&](const Off (&o)[kCopiesPerHalf], const int8_t* codes,
                        const _Float16* scales, int img_codes, int img_scales) {
#pragma unroll
    for (int i = 0; i < kStage / 4; ++i) {
      if constexpr (WIDE)
        dma16_wide(codes + o[i], lds0 + img_codes + 1024 * i);
      else
        dma16(codes, o[i], lds0 + img_codes + 1024 * i);
    }
    if constexpr (WIDE)
      dma4_wide(reinterpret_cast<const uint8_t*>(scales) + o[kStage / 4], lds0 + img_scales);
    else
      dma4(scales, o[kStage / 4], lds0 + img_scales);
  };
  // ids of chunk k into the image (positions past the row read its last
  // id, which the softmax masks)
  auto issue_ids = [&](int k) {
    const int p = min(k * kChunk + lane, nsel - 1);
    dma4(ids_row, 4 * p, lds0 + kImgIds);
  };

  f32x4 oacc[16];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Copy schedule.  K of stage s + 1 is started in stage s's K phase, V of
  // stage s + 1 in its V phase, each from offsets computed one phase pair
  // earlier (the shuffles' latency hides behind a PV).  The ids of chunk
  // k + 2 are copied in stage 2 k's V phase, just before V of stage 2 k + 1,
  // and read out in stage 2 k + 2's.  The wavefront's first two chunks come
  // from plain loads.
  auto position = [&](int k) { return min(k * kChunk + lane, nsel - 1); };
  int ids_next;
  int cells[kCopiesPerHalf];  // cells of the next stage's copies
  Off offs[kCopiesPerHalf];
  {
    const int ids0 = identity ? position(k_begin) : clamp_cell(ids_row[position(k_begin)]);
    ids_next = identity ? position(k_begin + 1) : clamp_cell(ids_row[position(k_begin + 1)]);
    // both loads complete before the first copy (the copies' waits count
    // copies only)
    asm volatile("" : : "v"(ids0), "v"(ids_next));
    cells_of(s_begin, ids0, cells);
    offsets_of(cells, offs);
    issue_half(offs, kq_g, ksc_g, kImgK, kImgKs);
    issue_half(offs, vq_g, vsc_g, kImgV, kImgVs);
    cells_of(s_begin + 1, ids0, cells);
  }

  for (int s = s_begin; s < s_end; ++s) {
    const bool more = s + 1 < s_end;
    const bool even = (s & 1) == 0;
    const int k = s >> 1;
    // ---- K phase: K of stage s into registers, K of stage s + 1 started.
    // Outstanding behind K of stage s: V of stage s, after the ids copy of
    // the previous stage's V phase when there was one.
    if (!even)
      wait_copies_10();
    else
      wait_copies_9();
    i32x4 kraw[2][4];
    u32x4 ks[2][2];  // scales of cells 16 mt + 4 j + r: dword 2 r + b / 2, half b % 2
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int row = stage_row(16 * mt + n);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int slot = (4 * b + j) ^ (row & 15);
        kraw[mt][b] = *reinterpret_cast<const i32x4*>(img + kImgK + row * kHeadDim + 16 * slot);
      }
      const uint8_t* sk = img + kImgKs + 8 * (16 * mt + 4 * j);
      ks[mt][0] = *reinterpret_cast<const u32x4*>(sk);
      ks[mt][1] = *reinterpret_cast<const u32x4*>(sk + 16);
    }
    if (more) offsets_of(cells, offs);
    wait_lds_reads();
    if (more) issue_half(offs, kq_g, ksc_g, kImgK, kImgKs);

    // ---- S^T = K Q^T: per 64-dim block, 256 I_hi + I_lo (< 2^29, exact)
    // times the cell's K scale of that block
    f32x4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const i32x4 zero = {0, 0, 0, 0};
        const i32x4 ih = mfma_i8(kraw[mt][b], qh[b], zero);
        const i32x4 ii = mfma_i8(kraw[mt][b], ql[b], ih << 8);  // 256 I_hi + I_lo
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t sw = ks[mt][r >> 1][2 * (r & 1) + (b >> 1)];
          const float sc = (float)as_h2(sw)[b & 1];
          acc[r] = __builtin_fmaf(sc, (float)ii[r], acc[r]);
        }
      }
      sacc[mt] = acc;
    }

    // ---- softmax over the stage (base 2, lazy reference max)
    float x[2][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = kStage * s + 16 * mt + 4 * j + r;
        x[mt][r] = (p < nsel) ? sacc[mt][r] * xs : -INFINITY;
        cmax = fmaxf(cmax, x[mt][r]);
      }
    cmax = wave_max_xor16_32(cmax);
    const bool grow = cmax > m_run + kLazyGrowth;
    if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) oacc[mt] *= alpha;
      m_run = m_new;
    }
    half8_t pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = fast_exp2(x[i >> 2][i & 3] - m_run);
      l_run += p;
      pb[i] = (_Float16)p;
    }

    // ---- V phase: V of stage s into registers, V of stage s + 1 started.
    // Outstanding behind V of stage s: K of stage s + 1 only.
    if (more)
      wait_copies_9();
    else
      wait_copies_0();
    u32x4 vrow[8];
    half2_t sp[4];  // V scales of the cell pairs (2 i, 2 i + 1), this lane's block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = (i < 4) ? (4 * j + i) : (16 + 4 * j + (i - 4));
      const int row = stage_row(c);
      vrow[i] = *reinterpret_cast<const u32x4*>(img + kImgV + row * kHeadDim +
                                                16 * (n ^ (row & 15)));
      sp[i >> 1][i & 1] = *reinterpret_cast<const _Float16*>(img + kImgVs + 8 * c + 2 * (n >> 2));
    }
    const bool new_chunk = even && k > k_begin;  // the ids of chunk k + 1 are due
    int ids_raw = 0;
    if (new_chunk) ids_raw = *reinterpret_cast<const int*>(img + kImgIds + 4 * lane);
    wait_lds_reads();
    if (new_chunk) ids_next = identity ? position(k + 1) : clamp_cell(ids_raw);
    if (more) {
      if (even) issue_ids(k + 2);
      issue_half(offs, vq_g, vsc_g, kImgV, kImgVs);
      // stage s + 2 lies in chunk k + 1 for either parity of s
      if (s + 2 < nst) cells_of(s + 2, ids_next, cells);
    }

    // ---- O^T += V^T P^T, one 32-cell k-step, 16 dim m-tiles
    static_for<16>([&](auto MT) {
      constexpr int mt = decltype(MT)::value;
      constexpr int dw = mt >> 2, by = mt & 3;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = as_u32(col_pair<by>(vrow[2 * i][dw], vrow[2 * i + 1][dw]) * sp[i]);
      const half8_t av = __builtin_bit_cast(half8_t, u32x4{w[0], w[1], w[2], w[3]});
      oacc[mt] = mfma16(av, pb, oacc[mt]);
    });
  }

  wait_copies_0();  // no copy into the image outlives the wave

  const float l_tot = wave_sum_xor16_32(l_run);
  if (!qvalid) return;
  if constexpr (PIECES) {
    // the piece's record: O unnormalised, m in natural-log units, l
    float* rec = a.part + (((int64_t)t * kcr + piece) * H + hq) * kRec;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int mt = 0; mt < 16; mt += 2)
        *reinterpret_cast<float2*>(rec + 64 * j + 16 * r + mt) = float2{oacc[mt][r], oacc[mt + 1][r]};
    if (j == 0) *reinterpret_cast<float2*>(rec + kHeadDim) = float2{m_run * kLn2, l_tot};
    return;
  }
  const float inv = 1.f / l_tot;
  _Float16* orow = a.out + ((int64_t)t * H + hq) * kHeadDim + 64 * j;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    half8_t h0, h1;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      h0[mt] = (_Float16)(oacc[mt][r] * inv);
      h1[mt] = (_Float16)(oacc[mt + 8][r] * inv);
    }
    *reinterpret_cast<half8_t*>(orow + 16 * r) = h0;
    *reinterpret_cast<half8_t*>(orow + 16 * r + 8) = h1;
  }
}

hipError_t launch_flash_rows(const RowArgs& args_in, bool split, int t_begin,
                             hipStream_t stream) {
  RowArgs a = args_in;
  if (split) t_begin = 0;
  a.n_items = split ? a.T * a.KC * a.G : (a.T - t_begin) * a.G;
  if (a.n_items <= 0) return hipSuccess;
  // the fused row kernel attends rows above budget only
  if (!split && (int64_t)a.pos0 + t_begin + 1 <= a.budget) return hipErrorInvalidValue;
  dim3 grid((a.n_items + 3) / 4), block(256);
  if (!split && kXcds % a.G == 0) {
    // kXcds / G workgroup slots per round serve each group, 4 rows apiece
    const int per = kXcds / a.G;
    const int wgs_per_group = (a.T - t_begin + 3) / 4;
    grid = dim3(kXcds * ((wgs_per_group + per - 1) / per));
  }
  if (split)
    flash_split_kernel<<<grid, block, 0, stream>>>(a);
  else if (a.n_cells <= (int64_t(1) << 24))
    flash_rows_staged_kernel<false, false><<<grid, block, 0, stream>>>(a);
  else
    flash_rows_staged_kernel<true, false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_flash_row_pieces(const RowArgs& args_in, hipStream_t stream) {
  RowArgs a = args_in;
  if (a.T <= 0) return hipSuccess;
  // the ids copies of rows under budget read the last row: it must be above
  if (a.cpr < 1 || !a.part || !a.ids || (int64_t)a.pos0 + a.T <= a.budget)
    return hipErrorInvalidValue;
  const int kcr = (a.KC + a.cpr - 1) / a.cpr;
  a.n_items = a.T * a.G * kcr;
  dim3 grid((a.n_items + 3) / 4), block(256);
  if (a.n_cells <= (int64_t(1) << 24))
    flash_rows_staged_kernel<false, true><<<grid, block, 0, stream>>>(a);
  else
    flash_rows_staged_kernel<true, true><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
