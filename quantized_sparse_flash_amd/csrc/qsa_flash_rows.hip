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
// This kernel serves every row kind: identity rows, rows with explicit ids
// (budget exceeded) and split mode.  Work mapping (gfx950, wave64):
//   * lane l: n = l % 16 is a query column (head n of the group, n < 12;
//     columns 12..15 carry zero queries), j = l / 16 a k-slot group;
//   * S^T[64 cells][16 queries] = K Q^T on v_mfma_f32_16x16x32_f16: A = K
//     (row = cell), B = Q^T, k = head dim.  Dim d of k-step s, slot (j, i)
//     is 64*(s/2) + 16*j + 8*(s%2) + i, so one 16-byte load per scale block
//     feeds two k-steps and each lane's codes share one K scale;
//   * the softmax runs on the S^T accumulators: every lane holds one query
//     and 16 cells, so row max/sum need only two cross-lane steps; the fused
//     mode keeps a lazy reference max (O and l are rescaled only when a
//     chunk max passes it by more than 2^8, so p stays below 2^8);
//   * O^T[256 dims][16 queries] += V^T P^T: B = P^T comes straight from the
//     S^T registers (the accumulator layout of two 16-cell tiles is exactly
//     the B layout of one 32-cell k-step); A = V^T uses dim d = 16*r + mt for
//     row r of m-tile mt, so a lane reads 16 contiguous codes of each of its
//     8 cells once and byte-selects them for all 16 m-tiles;
//   * int8 -> fp16 is one SDWA convert per element, then a packed fp16
//     multiply by the cell's scale (k and v rounded to fp16 once).
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


// Two waves per SIMD (at most 256 registers each): the gathers are latency-
// bound, and the second wave's loads overlap the first one's arithmetic.
template <bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void flash_rows_kernel(RowArgs a) {
  const int lane = threadIdx.x & 63;
  const int G = a.G, H = G * kHpg;
  int t, g, k_only = 0;
  if (SPLIT) {
    // wave-uniform: every per-row value below lives in scalar registers
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (item >= a.n_items) return;
    g = item % G;
    k_only = (item / G) % a.KC;
    t = item / (G * a.KC);
  } else if (kXcds % G == 0) {
    // workgroups are dealt to the XCDs round robin: XCD x serves group
    // x % G only, so each XCD's L2 caches one group's cells
    const int per = kXcds / G;
    const int b = blockIdx.x, x = b % kXcds;
    const int r = __builtin_amdgcn_readfirstlane(4 * ((b / kXcds) * per + x / G) +
                                                 (threadIdx.x >> 6));
    g = x % G;
    if (r >= a.n_items / G) return;
    t = a.T - 1 - r;  // longest rows first
  } else {
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (item >= a.n_items) return;
    g = item % G;
    t = a.T - 1 - item / G;  // longest rows first
  }
  const int64_t nkv = (int64_t)a.pos0 + t + 1;
  const bool explicit_ids = nkv > a.budget;
  const int nsel = explicit_ids ? a.budget : (int)nkv;
  const int nch = (nsel + kChunk - 1) / kChunk;
  if (SPLIT && k_only >= nch) return;

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
  const int32_t* ids_row = explicit_ids ? a.ids + ((int64_t)t * G + g) * a.budget : nullptr;

  f32x4 oacc[16];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int k_begin = SPLIT ? k_only : 0;
  const int k_end = SPLIT ? k_only + 1 : nch;
  float m_chunk = 0.f, l_chunk = 0.f;
  // id of chunk position `lane`, fetched one chunk ahead and clamped when
  // used; the row's ids sit behind a range-checked buffer (0 past the row)
  const __amdgpu_buffer_rsrc_t ids_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(explicit_ids ? ids_row : a.ids), (short)0,
      explicit_ids ? 4 * nsel : 0, kBufferFlags);
  auto raw_id = [&](int k) -> int {
    const int p = k * kChunk + lane;
    if (!explicit_ids) return p < nsel ? p : 0;
    return __builtin_amdgcn_raw_buffer_load_b32(ids_rs, 4 * p, 0, 0);
  };
  auto clamp_cell = [&](int c) -> int {
    c = c < 0 ? 0 : c;
    return (int64_t)c >= a.n_cells ? (int)(a.n_cells - 1) : c;
  };
  int next_raw = raw_id(k_begin);
  for (int k = k_begin; k < k_end; ++k) {
    const int cbase = k * kChunk;
    const int my_cell = clamp_cell(next_raw);
    next_raw = raw_id(k + 1);

    // V codes and scales of k-step kk: lane (n, j) takes dims 16n..16n+15
    // of the cells at positions 4j + i and 16 + 4j + i of the 32-cell half
    auto load_v = [&](int kk, u32x4 (&vrow)[8], uint32_t (&vs)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pos = 32 * kk + ((i < 4) ? (4 * j + i) : (16 + 4 * j + (i - 4)));
        const int cell = __shfl(my_cell, pos);
        vrow[i] = *reinterpret_cast<const u32x4*>(vq_g + (int64_t)cell * kHeadDim + 16 * n);
        vs[i] = *reinterpret_cast<const uint16_t*>(vsc_g + (int64_t)cell * kNBlk + (n >> 2));
      }
    };
    // split mode handles one chunk per wave: its V loads go out with K's
    // (one memory round trip instead of two); the fused loop keeps V's
    // registers free until the scores are done
    u32x4 vrow_s[2][8];
    uint32_t vs_s[2][8];
    if constexpr (SPLIT) {
      load_v(0, vrow_s[0], vs_s[0]);
      load_v(1, vrow_s[1], vs_s[1]);
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

    // ---- softmax over the chunk (base 2)
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
    float mref;
    if (SPLIT) {
      mref = cmax;
    } else {
      // the reference max moves only when a query's chunk max passes it by
      // more than 2^kLazyGrowth; p may then exceed 1 by at most that factor
      const bool grow = cmax > m_run + kLazyGrowth;
      if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
        const float m_new = grow ? cmax : m_run;
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) oacc[mt] *= alpha;
        m_run = m_new;
      }
      mref = m_run;
    }
    float lsum = 0.f;
    half8_t pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = fast_exp2(x[2 * kk + (i >> 2)][i & 3] - mref);
        lsum += p;
        pb[kk][i] = (_Float16)p;
      }
    }
    if (SPLIT) {
      m_chunk = cmax;
      l_chunk = wave_sum_xor16_32(lsum);
    } else {
      l_run += lsum;
    }

    // ---- O^T += V^T P^T, two 32-cell k-steps, 16 dim m-tiles
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 vrow[8];
      uint32_t vs[8];
      if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          vrow[i] = vrow_s[kk][i];
          vs[i] = vs_s[kk][i];
        }
      } else {
        load_v(kk, vrow, vs);
      }
      half2_t sp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[i] = as_h2(vs[2 * i] | (vs[2 * i + 1] << 16));
      static_for<16>([&](auto MT) {
        constexpr int mt = decltype(MT)::value;
        constexpr int dw = mt >> 2, by = mt & 3;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = as_u32(col_pair<by>(vrow[2 * i][dw], vrow[2 * i + 1][dw]) * sp[i]);
        const half8_t av = __builtin_bit_cast(half8_t, u32x4{w[0], w[1], w[2], w[3]});
        oacc[mt] = mfma16(av, pb[kk], oacc[mt]);
      });
    }
  }

  if (!SPLIT) {
    const float l_tot = wave_sum_xor16_32(l_run);
    if (!qvalid) return;
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
  } else {
    if (!qvalid) return;
    float* rec = a.part + (((int64_t)t * a.KC + k_only) * H + hq) * kRec;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int mt = 0; mt < 16; mt += 2) {
        const float2 v = {oacc[mt][r], oacc[mt + 1][r]};
        *reinterpret_cast<float2*>(rec + 64 * j + 16 * r + mt) = v;
      }
    }
    if (j == 0) *reinterpret_cast<float2*>(rec + kHeadDim) = float2{m_chunk * kLn2, l_chunk};
  }
}

hipError_t launch_flash_rows(const RowArgs& args_in, bool split, int t_begin,
                             hipStream_t stream) {
  RowArgs a = args_in;
  if (split) t_begin = 0;
  a.n_items = split ? a.T * a.KC * a.G : (a.T - t_begin) * a.G;
  if (a.n_items <= 0) return hipSuccess;
  dim3 grid((a.n_items + 3) / 4), block(256);
  if (!split && kXcds % a.G == 0) {
    // kXcds / G workgroup slots per round serve each group, 4 rows apiece
    const int per = kXcds / a.G;
    const int wgs_per_group = (a.T - t_begin + 3) / 4;
    grid = dim3(kXcds * ((wgs_per_group + per - 1) / per));
  }
  if (split)
    flash_rows_kernel<true><<<grid, block, 0, stream>>>(a);
  else
    flash_rows_kernel<false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qsa
