// qsa_flash_tile.hip -- fused attention for tokens under the budget, tiled
// over 10 consecutive tokens of one KV group.
//
// Pages: "round 6 track b - qsa flash" (delivered change: a token that sees
// at most `budget` cells attends to all of them, ids derived in the kernel;
// each selected cell's two scale vectors are staged once) and "opus_r9_qsa"
// (what changed: 64-cell chunks, S scaled by 1/16, online softmax, fp16 P
// accumulated against V).
//
// Under identity selection token t attends cells [0, pos0+t], a prefix of
// what token t+1 attends, so every token of the prompt chunk reads the same
// cells.  The path therefore dequantises each visible cell once per layer
// and then runs a plain fp16 flash kernel over the result:
//
//   dequant_chunks_kernel  one workgroup per (group, 64-cell chunk): int8
//     codes x fp16 scale -> fp16 (one SDWA convert + half a packed multiply
//     per element: the value is rounded to fp16 once, as when the pages'
//     kernel fills its K/V tiles), laid out in LDS as the 64 KB image the
//     attention kernel consumes, then streamed to the workspace with
//     coalesced 16-byte stores:  K [cell][dim] with 16-byte groups
//     XOR-swizzled by cell, and V^T [dim][slot] with cells permuted inside
//     each 32-cell half (so that one 16-byte read yields the eight cells an
//     MFMA k-slot group needs) and 8-byte groups XOR-swizzled by dim.  Cells
//     past the last visible one are zero.
//
//   flash_tile_kernel  one workgroup per (group, 10 tokens): 120 queries
//     (10 tokens x 12 heads) on 4 waves x 32 query slots.  Chunk images
//     stream from L2 straight into one of two LDS buffers
//     (global_load_lds_dwordx4, one chunk ahead, no registers held); each
//     wave computes S^T[64 cells][32 queries] on v_mfma_f32_16x16x32_f16
//     (A = K from LDS, B = Q^T held in registers), runs the online softmax on
//     the accumulator registers (each lane owns one query), takes the first
//     chunk's max as its reference (later chunks never rescale O; a rare
//     workgroup-wide fallback pass handles scores that outgrow it by 2^15),
//     and accumulates O^T[256 dims][32 queries] += V^T P^T with P taken
//     straight from the S^T registers.
//
// Workgroup i takes KV group i % G; with G = 2 and workgroups dealt to the
// 8 XCDs round robin, each XCD's L2 holds one group's images only.
#include <utility>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

constexpr int kNT = 2;                      // 16-query N-tiles per wave
constexpr int kSlots = 4 * 16 * kNT;        // query slots per workgroup
constexpr int kTileTokens = kSlots / kHpg;  // whole tokens per workgroup (10)
constexpr float kMaxGrowth = 15.0f;         // log2 headroom above the reference max
constexpr int kImgK = kChunk * kHeadDim * 2;  // bytes of the K image (32 KB)
constexpr int kImgV = kHeadDim * kChunk * 2;  // bytes of the V^T image (32 KB)
constexpr int kImg = kImgK + kImgV;           // bytes per (group, chunk) image
constexpr int kCopyOps = kImg / 4 / 1024;     // 1 KB copies per wave per chunk (16)

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// 64 lanes x 16 bytes from global memory straight into LDS: lane i's 16
// bytes at `g` land at LDS byte lds + 16 i (lds must be wave-uniform).
// Written as inline asm so that the compiler does not track the LDS write:
// it would otherwise make every later LDS read wait for the copy to
// complete, which serialises the prefetch with the math.  Completion is
// awaited explicitly with wait_copies_but(), before a barrier publishes the
// data.  The asm loads M0 itself; nothing else in this kernel uses M0 (DS
// instructions on gfx9+ do not read it), so the clobber is harmless here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* g, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most n of this wave's vector-memory operations (the copies
// above, issued in order) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory");
}
__device__ __forceinline__ void wait_copies_but(int n) {
  if (n == 0) wait_vmcnt<0>(); else wait_vmcnt<kCopyOps>();
}

// Max over the four 16-lane groups of a wave (lanes n, n+16, n+32, n+48),
// on the VALU: v_permlane16_swap pairs rows {0,1} and {2,3}, then
// v_permlane32_swap pairs the two halves.
__device__ __forceinline__ float lane_group_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Workgroup barrier without the memory wait __syncthreads() adds; the
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Byte offset of the 16-byte group `grp` (8 dims) of K row `cell`.
__device__ __forceinline__ int kimg_off(int cell, int grp) {
  return cell * (kHeadDim * 2) + 16 * (grp ^ (cell & 7));
}
// Slot of chunk cell c in a V^T row: inside each 32-cell half, cells
// {4j..4j+3, 16+4j..16+4j+3} become the consecutive slots 8j..8j+7 (the k
// slots of lane group j in one 32-cell MFMA k-step).
__device__ __forceinline__ int vperm(int c) {
  const int kk = c >> 5, cc = c & 31;
  return 32 * kk + 8 * ((cc & 15) >> 2) + 4 * (cc >> 4) + (cc & 3);
}
// Byte offset (inside the chunk image) of the 8-byte group `grp` (4 slots)
// of V^T row d; the XOR is even, so 16-byte pairs of groups stay adjacent.
__device__ __forceinline__ int vimg_off(int d, int grp) {
  return kImgK + d * (kChunk * 2) + 8 * (grp ^ (2 * ((d & 7) ^ ((d >> 4) & 7))));
}

}  // namespace

// ---------------------------------------------------------------- dequant
__global__ __launch_bounds__(256) void dequant_chunks_kernel(RowArgs a, int n_needed,
                                                             int nchunks, uint8_t* ws) {
  __shared__ __attribute__((aligned(16))) uint8_t img[kImg];
  const int tid = threadIdx.x;
  const int g = blockIdx.x / nchunks, k = blockIdx.x % nchunks;
  const int cbase = k * kChunk;
  const int8_t* kq_g = a.kq + (int64_t)g * a.n_cells * kHeadDim;
  const int8_t* vq_g = a.vq + (int64_t)g * a.n_cells * kHeadDim;
  const _Float16* ksc_g = a.ksc + (int64_t)g * a.n_cells * kNBlk;
  const _Float16* vsc_g = a.vsc + (int64_t)g * a.n_cells * kNBlk;

  // K: units (cell, 16 dims): cell tid/16 + 16i, segment tid%16
  {
    const int seg = tid & 15;
    u32x4 raw[4];
    uint32_t sr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (tid >> 4) + 16 * i;
      const int cell = min(cbase + c, n_needed - 1);
      raw[i] = *reinterpret_cast<const u32x4*>(kq_g + (int64_t)cell * kHeadDim + 16 * seg);
      sr[i] = *reinterpret_cast<const uint16_t*>(ksc_g + (int64_t)cell * kNBlk + (seg >> 2));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (tid >> 4) + 16 * i;
      const bool live = cbase + c < n_needed;
      const half2_t sc = as_h2(live ? (sr[i] | (sr[i] << 16)) : 0u);
      uint32_t o[8];
      dq4(raw[i].x, sc, o[0], o[1]);
      dq4(raw[i].y, sc, o[2], o[3]);
      dq4(raw[i].z, sc, o[4], o[5]);
      dq4(raw[i].w, sc, o[6], o[7]);
      *reinterpret_cast<u32x4*>(img + kimg_off(c, 2 * seg)) = u32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4*>(img + kimg_off(c, 2 * seg + 1)) = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
  // V: units (4 cells 4*cg.., 16 dims 16*dg..), transposed into V^T rows
  {
    const int dg = tid & 15, cg = tid >> 4;
    u32x4 raw[4];
    uint32_t sr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cell = min(cbase + 4 * cg + i, n_needed - 1);
      raw[i] = *reinterpret_cast<const u32x4*>(vq_g + (int64_t)cell * kHeadDim + 16 * dg);
      const bool live = cbase + 4 * cg + i < n_needed;
      sr[i] = live ? *reinterpret_cast<const uint16_t*>(vsc_g + (int64_t)cell * kNBlk + (dg >> 2))
                   : 0u;
    }
    const half2_t s01 = as_h2(sr[0] | (sr[1] << 16));
    const half2_t s23 = as_h2(sr[2] | (sr[3] << 16));
    const int grp = vperm(4 * cg) >> 2;
    auto put = [&](auto E, int d, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
      constexpr int e = decltype(E)::value;  // byte inside the dwords
      const uint32_t lo = as_u32(col_pair<e>(w0, w1) * s01);
      const uint32_t hi = as_u32(col_pair<e>(w2, w3) * s23);
      *reinterpret_cast<u32x2*>(img + vimg_off(d, grp)) = u32x2{lo, hi};
    };
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const uint32_t w0 = raw[0][dw], w1 = raw[1][dw], w2 = raw[2][dw], w3 = raw[3][dw];
      const int d = 16 * dg + 4 * dw;
      put(std::integral_constant<int, 0>{}, d + 0, w0, w1, w2, w3);
      put(std::integral_constant<int, 1>{}, d + 1, w0, w1, w2, w3);
      put(std::integral_constant<int, 2>{}, d + 2, w0, w1, w2, w3);
      put(std::integral_constant<int, 3>{}, d + 3, w0, w1, w2, w3);
    }
  }
  __syncthreads();
  uint8_t* dst = ws + (int64_t)blockIdx.x * kImg;
#pragma unroll
  for (int i = 0; i < kImg / 16 / 256; ++i) {
    const int off = 16 * (tid + 256 * i);
    *reinterpret_cast<u32x4*>(dst + off) = *reinterpret_cast<const u32x4*>(img + off);
  }
}

// ---------------------------------------------------------------- attention
__global__ __launch_bounds__(256, 1) void flash_tile_kernel(RowArgs a, int t_count, int nchunks,
                                                            const uint8_t* ws) {
  __shared__ __attribute__((aligned(16))) uint8_t bufs[2 * kImg];  // chunk k in half k & 1
  __shared__ int s_redo;  // set when the fast pass must be redone exactly
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.G, H = G * kHpg;
  const int n_blocks = (t_count + kTileTokens - 1) / kTileTokens;
  // longest blocks first; consecutive workgroups alternate KV groups
  const int g = blockIdx.x % G;
  const int blk = n_blocks - 1 - blockIdx.x / G;
  const int t0 = blk * kTileTokens;
  const int t_last = min(t0 + kTileTokens, t_count) - 1;
  const int nkv_min = a.pos0 + t0 + 1;  // cells every token of the block sees
  const int nkv_max = a.pos0 + t_last + 1;
  const int nch = (nkv_max + kChunk - 1) / kChunk;
  const uint8_t* img_g = ws + (int64_t)g * nchunks * kImg;

  const int n = lane & 15, j = lane >> 4;

  // ---- per-lane queries: N-tile nt, column n -> query slot of the workgroup
  int nkv_q[kNT];
  bool qvalid[kNT];
  int qt[kNT], qh[kNT];
  half8_t qf[kNT][8];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int q = 16 * kNT * w + 16 * nt + n;
    const int t = t0 + q / kHpg;
    qt[nt] = t;
    qh[nt] = g * kHpg + q % kHpg;
    qvalid[nt] = q < kTileTokens * kHpg && t <= t_last;
    nkv_q[nt] = qvalid[nt] ? a.pos0 + t + 1 : 1;
    const _Float16* qrow = a.q + ((int64_t)(qvalid[nt] ? t : t0) * H + qh[nt]) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int d0 = 64 * (s >> 1) + 16 * j + 8 * (s & 1);
      qf[nt][s] = *reinterpret_cast<const half8_t*>(qrow + d0);
    }
  }

  // ---- chunk image k -> dbuf: wave w moves bytes [16 KB w, 16 KB (w+1))
  auto issue_copy = [&](int k, uint8_t* dbuf) {
    const uint8_t* src = img_g + (int64_t)k * kImg + w * (kImg / 4) + 16 * lane;
    const uint32_t dst = lds_addr(dbuf) + w * (kImg / 4);
#pragma unroll
    for (int i = 0; i < kCopyOps; ++i) copy16_to_lds(src + 1024 * i, dst + 1024 * i);
  };

  // One pass over the block's chunks.  Chunk k is read from its half of
  // `bufs` while chunk k+1 lands in the other.  Barriers are bare s_barrier:
  // __syncthreads() would also wait for every outstanding global access, i.e.
  // for the copy just issued.  Each wave consumes its LDS reads before a
  // barrier, and waits for its own copies (vmcnt) before the barrier that
  // publishes them.
  //
  // Softmax reference.  Fast pass (SAFE = false): chunk 0 sets each query's
  // reference max exactly (O is still zero); later chunks keep it, so O is
  // never rescaled.  P = 2^(x - m) then stays below 2^kMaxGrowth unless a
  // later score exceeds the reference by more than that; each lane records
  // whether one did, and the workgroup votes at the end.  Safe pass (SAFE =
  // true, only after such a vote): the exact online softmax, the running
  // max updated every chunk and O rescaled when it moves.  Either way the
  // result after the final division by l is the same softmax.
  auto run = [&](auto SAFE_T) -> bool {
    constexpr bool SAFE = decltype(SAFE_T)::value;
    f32x4 oacc[kNT][16];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) oacc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[kNT], l_run[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      m_run[nt] = -INFINITY;
      l_run[nt] = 0.f;
    }
    bool over = false;

    issue_copy(0, bufs);
    for (int k = 0; k < nch; ++k) {
      wg_barrier();  // every wave is done with chunk k-1, whose half gets chunk k+1
      if (k + 1 < nch) {
        issue_copy(k + 1, bufs + ((k + 1) & 1) * kImg);
        wait_copies_but(kCopyOps);  // chunk k landed; chunk k+1 may be in flight
      } else {
        wait_copies_but(0);
      }
      wg_barrier();  // chunk k landed for every wave
      const uint8_t* kb = bufs + (k & 1) * kImg;
      const int cbase = k * kChunk;

      // ---- S^T = K Q^T: k-step outer, 4 cell m-tiles x 2 query N-tiles inner
      f32x4 sacc[kNT][4];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sacc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        half8_t af[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *reinterpret_cast<const half8_t*>(
              kb + kimg_off(16 * mt + n, 8 * (s >> 1) + 2 * j + (s & 1)));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) sacc[nt][mt] = mfma16(af[mt], qf[nt][s], sacc[nt][mt]);
      }

      // ---- scores to plain registers; masking (cells past a token's n_kv)
      // only where the chunk reaches past the block's first token, against a
      // per-lane limit so that the cell offsets are immediates
      float sv[kNT][16];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[nt][4 * mt + r] = sacc[nt][mt][r];
      if (cbase + kChunk > nkv_min) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const int lim = nkv_q[nt] - cbase - 4 * j;  // cell 16mt+4j+r valid iff 16mt+r < lim
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * mt + r >= lim) sv[nt][4 * mt + r] = -INFINITY;
        }
      }
      float lmax[kNT];  // this lane's max over its 16 cells, raw score units
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const float c0 = fmaxf(fmaxf(sv[nt][0], sv[nt][1]), fmaxf(sv[nt][2], sv[nt][3]));
        const float c1 = fmaxf(fmaxf(sv[nt][4], sv[nt][5]), fmaxf(sv[nt][6], sv[nt][7]));
        const float c2 = fmaxf(fmaxf(sv[nt][8], sv[nt][9]), fmaxf(sv[nt][10], sv[nt][11]));
        const float c3 = fmaxf(fmaxf(sv[nt][12], sv[nt][13]), fmaxf(sv[nt][14], sv[nt][15]));
        lmax[nt] = fmaxf(fmaxf(c0, c1), fmaxf(c2, c3));
      }
      if constexpr (SAFE) {
        bool grew = false;
        float mnew[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          mnew[nt] = fmaxf(m_run[nt], lane_group_max(lmax[nt]) * kScoreScaleLog2);
          grew |= mnew[nt] > m_run[nt];
        }
        if (__builtin_amdgcn_ballot_w64(grew) != 0ull) {
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            const float alpha = fast_exp2(m_run[nt] - mnew[nt]);
            l_run[nt] *= alpha;
#pragma unroll
            for (int mt = 0; mt < 16; ++mt) oacc[nt][mt] *= alpha;
            m_run[nt] = mnew[nt];
          }
        }
      } else {
        if (k == 0) {
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            m_run[nt] = lane_group_max(lmax[nt]) * kScoreScaleLog2;  // finite: cell 0 is valid
        } else {
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            over |= lmax[nt] * kScoreScaleLog2 > m_run[nt] + kMaxGrowth;
        }
      }

      // ---- P and O^T += V^T P^T, one 32-cell half (k-step kk) at a time, so
      // the exponentials of the second half can overlap the first half's MFMAs
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        half8_t pb[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const float nm = -m_run[nt];
          float lsum = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = fast_exp2(__builtin_fmaf(sv[nt][8 * kk + i], kScoreScaleLog2, nm));
            lsum += p;
            pb[nt][i] = (_Float16)p;
          }
          l_run[nt] += lsum;
        }
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) {
          const half8_t av =
              *reinterpret_cast<const half8_t*>(kb + vimg_off(16 * mt + n, 8 * kk + 2 * j));
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) oacc[nt][mt] = mfma16(av, pb[nt], oacc[nt][mt]);
        }
      }
    }

    if constexpr (!SAFE) {
      // workgroup vote: any score beyond the reference by more than
      // 2^kMaxGrowth anywhere in the block sends the whole block to the safe
      // pass (its result would still be finite, but P could have overflowed)
      if (__builtin_amdgcn_ballot_w64(over) != 0ull && lane == 0) s_redo = 1;
      __syncthreads();
      if (s_redo) return true;
    }

    // ---- finalise: O / l -> fp16; lane (n, j) holds dims 16*mt + 4*j + r
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float l_tot = wave_sum_xor16_32(l_run[nt]);
      if (!qvalid[nt]) continue;
      const float inv = 1.f / l_tot;
      _Float16* orow = a.out + ((int64_t)qt[nt] * H + qh[nt]) * kHeadDim + 4 * j;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        half4_t h;
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = (_Float16)(oacc[nt][mt][r] * inv);
        *reinterpret_cast<half4_t*>(orow + 16 * mt) = h;
      }
    }
    return false;
  };

  // Q is in registers before any copy is issued: a compiler-visible wait, so
  // that no count-based wait for the Q loads is left inside the loop (it
  // would also wait for the copies, which the compiler does not count)
  if (tid == 0) s_redo = 0;
  __builtin_amdgcn_s_waitcnt(0);
  if (run(std::false_type{})) run(std::true_type{});
}

int64_t tile_workspace_bytes(int G, int t_count, int pos0) {
  if (t_count <= 0) return 0;
  const int64_t n_needed = (int64_t)pos0 + t_count;  // cells the last identity token sees
  const int64_t nchunks = (n_needed + kChunk - 1) / kChunk;
  return (int64_t)G * nchunks * kImg;
}

hipError_t launch_flash_tile(const RowArgs& a, int t_count, void* ws, hipStream_t stream) {
  if (t_count <= 0) return hipSuccess;
  const int n_needed = a.pos0 + t_count;
  const int nchunks = (n_needed + kChunk - 1) / kChunk;
  uint8_t* img = static_cast<uint8_t*>(ws);
  dequant_chunks_kernel<<<dim3(a.G * nchunks), dim3(256), 0, stream>>>(a, n_needed, nchunks, img);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_blocks = (t_count + kTileTokens - 1) / kTileTokens;
  flash_tile_kernel<<<dim3(n_blocks * a.G), dim3(256), 0, stream>>>(a, t_count, nchunks, img);
  return hipGetLastError();
}

}  // namespace qsa
