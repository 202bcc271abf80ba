// qsa_flash_tile.hip -- fused attention for tokens under the budget, tiled
// over 128 consecutive queries (the (token, head) pairs in order) of one KV
// group.
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
//   dequant_chunks_kernel  one one-wave workgroup per (group, 64-cell chunk,
//     32-cell half, V^T slot group of the half): int8 code x fp16
//     scale -> fp16 (the value is rounded to fp16
//     once, as when the pages' kernel fills its K/V tiles), written to the
//     workspace as the two 32 KB images the attention kernel copies verbatim
//     into LDS:
//       K    [64 cells][256 dims], the 16-byte group g of cell c's row at
//            position g ^ (c & 15);
//       V^T  [256 dims][64 slots]: 16-byte group 4 kk + j (kk = 32-cell half,
//            j < 4) holds the cells 32 kk + 16 (e / 4) + 4 j + e % 4 for
//            e = 0..7 (the eight cells an MFMA k-slot group needs, see
//            below), and group g of dim d's row sits at position
//            g ^ ((d >> 1) & 7).
//     Both swizzles make the 16-byte MFMA operand reads conflict-free for
//     any 16 consecutive rows.  Cells past the last visible one are zero.
//
//   flash_tile_kernel  one workgroup per (group, block of 128 consecutive
//     queries of the group's (token, head) pairs, about 10.7 tokens) on 8
//     waves x 16 query slots, two waves per SIMD, so that one wave's softmax
//     runs on the VALU while the other's products occupy the matrix core;
//     every slot holds a query but in a group's last block.  When that grid
//     would not cover the 256 CUs (short prompts), workgroups of 4 waves
//     take 64 queries each: twice the workgroups, each running its chunks
//     about twice as fast on one wave per SIMD.  Products on v_mfma_f32_16x16x32_f16
//     with queries in the N dimension:
//       S^T[64 cells][16 queries] = K Q^T   (A = K from LDS, B = Q^T held in
//                                            registers for the whole block)
//       O^T[256 dims][16 queries] += V^T P^T (A = V^T from LDS, B = P^T taken
//                                            straight from the S^T registers)
//     Lane l owns query l % 16 and the cells 16 mt + 4 (l / 16) + i of the
//     chunk (mt, i < 4): row max and sum take two cross-lane steps, and the
//     S^T registers of two consecutive 16-cell tiles are exactly the B
//     operand of one 32-cell PV k-step once V^T uses the slot order above.
//
//     Software pipeline, one barrier per chunk: each wave issues chunk k+1's
//     score MFMAs before chunk k's softmax, then chunk k's PV.  K and V^T
//     images have separate double buffers: at chunk k the kernel reads K(k+1)
//     and V(k) while K(k+2) and V(k+1) stream from L2 into the free halves
//     (global_load_lds_dwordx4, no registers held), issued from inside the
//     chunk's stage sequence rather than at its start.
//
//     Softmax reference.  The first chunk sets each query's reference max
//     exactly; later chunks keep it, so O is never rescaled.  P = 2^(x - m)
//     may then exceed 1 when a later score passes the reference; every P is
//     at most l (their fp32 sum), so l < 65504 at the end proves that no P
//     overflowed fp16.  Otherwise (rare: scores far above chunk 0's) the
//     workgroup votes to recompute the block by an exact online-softmax
//     pass that moves the running max and rescales O (one chunk per step,
//     no overlap: it is rare, and lean in registers).  Either way the result
//     after the final division by l is the same softmax.
//
//     Output.  The fast pass stages each wave's O^T tile, as fp16 rows, in
//     the idle chunk buffers and writes it with 16-byte non-temporal
//     stores, two whole 512-byte output rows per store instruction.
//
// Workgroup i takes KV group i % G; with G = 2 and workgroups dealt to the
// 8 XCDs round robin, each XCD's L2 holds one group's images only.
#include <type_traits>

#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

constexpr int kQpw = 16;  // query slots per wave
// Queries per workgroup of `waves` waves: 128 with 8 waves, 64 with 4.  A
// block takes that many consecutive queries of the group's (token, head)
// pairs in order, so every query slot is used but in a group's last block.
__host__ __device__ constexpr int tile_queries(int waves) { return kQpw * waves; }
__host__ __device__ inline int tile_blocks(int t_count, int waves) {
  return (t_count * kHpg + tile_queries(waves) - 1) / tile_queries(waves);
}
// Chunks block b attends: the cells its last token sees, in 64-cell chunks.
__host__ __device__ inline int block_chunks(int b, int t_count, int pos0, int waves) {
  const int q_last = min((b + 1) * tile_queries(waves), t_count * kHpg) - 1;
  return (pos0 + q_last / kHpg + 1 + kChunk - 1) / kChunk;
}
// First chunk of piece p of a block of nch chunks split into k pieces.
__host__ __device__ constexpr int piece_start(int nch, int p, int k) { return p * nch / k; }
constexpr int kMaxPieces = 3;  // pieces per split block
// MI355X compute units: below this many 8-wave workgroups the grid would
// leave CUs idle, and 4-wave workgroups of half as many tokens are used.
constexpr int kCus = 256;
constexpr float kP16Max = 65504.0f;         // largest finite fp16
constexpr int kHalf = kChunk * kHeadDim * 2;  // bytes of one K or V^T image (32 KB)
constexpr int kImg = 2 * kHalf;               // bytes per (group, chunk) in the workspace
constexpr int kHalfCells = kChunk / 2;           // cells per PV k-step
// A split piece's partial result in the workspace: its O (unnormalised,
// fp32, one 16-byte group per (wave, M-tile, lane) in that order, as the
// registers hold it), then (m, l) per query slot.
__host__ __device__ constexpr int part_floats(int waves) {
  return tile_queries(waves) * kHeadDim + 2 * tile_queries(waves);
}

// Where a launch's split pieces keep their counters and partials.
struct TileSplit {
  int n_split;  // blocks split per group: the longest ones
  int pieces;   // workgroups per split block (2 .. kMaxPieces)
  int* cnt;     // [G * n_split] arrival counters, zero between launches
  float* part;  // [G * n_split][pieces][part_floats(waves)]
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) const half8_t lds_half8_t;

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// 64 lanes x 16 bytes from global memory straight into LDS: lane i's 16
// bytes at base + voff (voff per lane, base wave-uniform) land at LDS byte
// lds + 16 i (lds must be wave-uniform).  Written as inline asm so that the
// compiler does not track the LDS write: it would otherwise make every later
// LDS read wait for the copy to complete, which serialises the prefetch with
// the math.  Completion is awaited explicitly (s_waitcnt vmcnt) before a
// barrier publishes the data.  The asm loads M0 itself; nothing else in this
// kernel uses M0 (DS instructions on gfx9+ do not read it), so the clobber is
// harmless here.  No immediate offset is used: on this copy the offset field
// moves the LDS destination as well as the global source.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until none of this wave's vector-memory operations is outstanding.
__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// Workgroup barrier without the memory wait __syncthreads() adds; the
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Max / sum over the four 16-lane groups of a wave (lanes n, n+16, n+32,
// n+48), on the VALU: v_permlane16_swap pairs rows {0,1} and {2,3}, then
// v_permlane32_swap pairs the two halves.
// (the asm swaps of qsa_device.h: the compiler's builtins for these swaps
// can hand one operation the same result twice)
__device__ __forceinline__ float lane_group_max(float v) { return wave_max_xor16_32(v); }
__device__ __forceinline__ float lane_group_sum(float v) { return wave_sum_xor16_32(v); }

// Byte offset of the 16-byte group `grp` (8 dims) of K row `cell`.
__device__ __forceinline__ int kimg_off(int cell, int grp) {
  return cell * (kHeadDim * 2) + 16 * (grp ^ (cell & 15));
}
// Byte offset of the 16-byte group `grp` (8 slots) of V^T row `d`.
__device__ __forceinline__ int vimg_off(int d, int grp) {
  return d * (kChunk * 2) + 16 * (grp ^ ((d >> 1) & 7));
}
// Cell (inside its 32-cell half) of V^T slot e of k-slot group j.
__host__ __device__ constexpr int vslot_cell(int j, int e) {
  return 16 * (e >> 2) + 4 * j + (e & 3);
}

}  // namespace

// ---------------------------------------------------------------- dequant
// One one-wave workgroup per (group, chunk, 32-cell half kk, j); it takes
// V^T slot group 4 kk + j, i.e. the eight cells 32 kk + 16 (e / 4) + 4 j + e % 4
// (e < 8) that fill one 16-byte slot group of every V^T row.  Lane i
// converts dims 4 i .. 4 i + 3 of those cells' V codes (one 4-byte load per
// cell) and writes the four slot groups; for K, lane i converts 32 dims of
// cell e = i / 8 and writes its four 16-byte groups.  Every load is issued
// before any use, and no LDS or barrier is needed; the four workgroups of
// one (group, chunk, kk) together write whole 64-byte pieces of each V^T
// row.  One wave per workgroup spreads the 8 G x chunks waves over more
// CUs than four-wave workgroups do (~1% shorter steps at T=1024); the grid
// is padded to whole groups of 32 workgroups, and the spare ones return.
__global__ __launch_bounds__(64) void dequant_chunks_kernel(RowArgs a, int n_needed,
                                                             int nchunks, uint8_t* ws, int* cnt,
                                                             int n_cnt) {
  const int lane = threadIdx.x & 63;
  // the attention launch's arrival counters start at zero
  if (blockIdx.x == 0)
    for (int i = lane; i < n_cnt; i += 64) cnt[i] = 0;
  // workgroups are dealt to the 8 XCDs round robin: the four waves j of one
  // (group, chunk, kk) get indices 8 apart, so they share an XCD's L2 and
  // their pieces of each V^T row merge there into whole lines
  const int pidx = ((blockIdx.x >> 5) << 3) | (blockIdx.x & 7);  // 2 gk + kk
  if (pidx >= 2 * a.G * nchunks) return;
  const int kk = pidx & 1, j = (blockIdx.x >> 3) & 3;
  const int u = 4 * kk + j;  // slot group
  const int gk = pidx >> 1;  // (group, chunk)
  const int g = gk / nchunks, k = gk % nchunks;
  uint8_t* img = ws + (int64_t)gk * kImg;
  const int64_t gbase = (int64_t)g * a.n_cells;
  auto cell_of = [&](int e) { return kHalfCells * kk + vslot_cell(j, e); };  // inside the chunk

  // ---- V: dims 4 lane .. +3 of the eight cells
  uint32_t vraw[8];
  uint16_t vbits[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int cell = k * kChunk + cell_of(e);
    const bool live = cell < n_needed;
    const int64_t row = gbase + (live ? cell : 0);
    vraw[e] = *reinterpret_cast<const uint32_t*>(a.vq + row * kHeadDim + 4 * lane);
    vbits[e] = live ? reinterpret_cast<const uint16_t*>(a.vsc)[row * kNBlk + (lane >> 4)]
                    : (uint16_t)0;
  }
  // ---- K: cell e = lane / 8, dims 32 (lane % 8) .. +31
  const int ke = lane >> 3, kseg = lane & 7;
  const int kc = cell_of(ke);
  const int kcell = k * kChunk + kc;
  const bool klive = kcell < n_needed;
  const int64_t krow = gbase + (klive ? kcell : 0);
  const u32x4 k0 = *reinterpret_cast<const u32x4*>(a.kq + krow * kHeadDim + 32 * kseg);
  const u32x4 k1 = *reinterpret_cast<const u32x4*>(a.kq + krow * kHeadDim + 32 * kseg + 16);
  const uint16_t kbits =
      klive ? reinterpret_cast<const uint16_t*>(a.ksc)[krow * kNBlk + (kseg >> 1)] : (uint16_t)0;

  auto code = [](uint32_t w, int byte) -> _Float16 { return (_Float16)(int8_t)(w >> (8 * byte)); };
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    half8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = code(vraw[e], m) * __builtin_bit_cast(_Float16, vbits[e]);
    *reinterpret_cast<half8_t*>(img + kHalf + vimg_off(4 * lane + m, u)) = v;
  }
  const _Float16 ks = __builtin_bit_cast(_Float16, kbits);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t w0 = (h < 2 ? k0 : k1)[2 * (h & 1)], w1 = (h < 2 ? k0 : k1)[2 * (h & 1) + 1];
    half8_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = code(w0, e) * ks;
      v[4 + e] = code(w1, e) * ks;
    }
    *reinterpret_cast<half8_t*>(img + kimg_off(kc, 4 * kseg + h)) = v;
  }
}

// ---------------------------------------------------------------- attention
// kSplit: the launch runs split blocks (sp); without it the chunk ranges
// are the whole blocks at compile time.
template <int kWaves, bool kSplit>
__global__ __launch_bounds__(kWaves * 64, 1) void flash_tile_kernel(RowArgs a, int t_count,
                                                                    int nchunks,
                                                                    const uint8_t* ws,
                                                                    TileSplit sp) {
  constexpr int kQpb = tile_queries(kWaves);
  constexpr int kCopyOps = kHalf / 1024 / kWaves;  // 1 KB copies per wave per image
  // K(c) lives in kv[(c - cb) & 1], V^T(c) in kv[2 + ((c - cb) & 1)]
  __shared__ __attribute__((aligned(16))) uint8_t kv[4 * kHalf];
  __shared__ int s_redo;  // set when the fast pass must be redone exactly
  __shared__ int s_flag;  // a split piece's arrival count
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.G, H = G * kHpg;
  const int n_blocks = tile_blocks(t_count, kWaves);
  // Longest blocks first; consecutive workgroups alternate KV groups.  The
  // n_split longest blocks of each group come first, each as sp.pieces
  // pieces over consecutive ranges of its chunks, G workgroups apart, that
  // merge their partial results; then the other blocks, one workgroup each.
  int g, blk, sb = -1, piece = 0;
  if (kSplit && blockIdx.x < sp.pieces * sp.n_split * G) {
    g = blockIdx.x % G;
    piece = (blockIdx.x / G) % sp.pieces;
    const int r = blockIdx.x / (sp.pieces * G);
    blk = n_blocks - 1 - r;
    sb = r * G + g;  // split block index: its counter and partial slots
  } else {
    const int n_first = kSplit ? sp.pieces * sp.n_split * G : 0;
    const int i = blockIdx.x - n_first;
    g = i % G;
    blk = n_blocks - 1 - (kSplit ? sp.n_split : 0) - i / G;
  }
  const int q0 = blk * kQpb;                                 // first query of the block
  const int q_last = min(q0 + kQpb, t_count * kHpg) - 1;     // last one
  const int t0 = q0 / kHpg;
  const int nkv_min = a.pos0 + t0 + 1;  // cells every token of the block sees
  const int nch = block_chunks(blk, t_count, a.pos0, kWaves);
  // this workgroup's chunks [cb, ce).  The host splits only blocks whose
  // tokens all see a cell of every piece's first chunk (64 cb < nkv_min),
  // so each piece's first chunk gives every query a finite softmax
  // reference.
  const int cb = (kSplit && sb >= 0) ? piece_start(nch, piece, sp.pieces) : 0;
  const int ce = (kSplit && sb >= 0) ? piece_start(nch, piece + 1, sp.pieces) : nch;
  const uint8_t* img_g = ws + (int64_t)g * nchunks * kImg;

  const int n = lane & 15, j = lane >> 4;

  // ---- this lane's query: slot kQpw w + n of the workgroup.  Slots past
  // the last query (a group's last block) compute as if they were its
  // first token and are never written.
  const int qs = q0 + kQpw * w + n;
  const bool qvalid = qs <= q_last;
  const int qt = qs / kHpg;
  const int qh = g * kHpg + qs % kHpg;
  const int nkv_q = qvalid ? a.pos0 + qt + 1 : nkv_min;
  // ---- LDS read addresses of this lane's operand fragments
  // K: row (cell) 16 mt + n, group 4 s + j; s = 4 v + u -> the XOR touches
  // the low 4 bits only, so v and mt are immediates
  uint32_t koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = lds_addr(kv) + kimg_off(n, 4 * u + j);
  // V^T: row (dim) 16 mt + n, group 4 kk + j
  uint32_t voff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) voff[kk] = lds_addr(kv) + 2 * kHalf + vimg_off(n, 4 * kk + j);

  // wave w copies bytes [4096 w, 4096 w + 4096) of an image: lane i's 16
  // bytes of each 1 KB piece at 16 i
  uint32_t copy_voff[kCopyOps];
#pragma unroll
  for (int i = 0; i < kCopyOps; ++i) copy_voff[i] = w * (kHalf / kWaves) + 1024 * i + 16 * lane;
  auto issue_copy = [&](const uint8_t* src, uint32_t dst) {
    const uint32_t d = dst + w * (kHalf / kWaves);
#pragma unroll
    for (int i = 0; i < kCopyOps; ++i) copy16_to_lds(src, copy_voff[i], d + 1024 * i);
  };
  auto copy_k = [&](int c) {
    issue_copy(img_g + (int64_t)c * kImg, lds_addr(kv) + ((c - cb) & 1) * kHalf);
  };
  auto copy_v = [&](int c) {
    issue_copy(img_g + (int64_t)c * kImg + kHalf, lds_addr(kv) + (2 + ((c - cb) & 1)) * kHalf);
  };

  // K(cb) streams in while Q loads; V(cb) and K(cb + 1) follow once both
  // are in (below), during the first chunk's scores
  copy_k(cb);

  half8_t qf[8];  // Q^T k-step s: dims 32 s + 8 j .. +7
  {
    const _Float16* qrow = a.q + ((int64_t)(qvalid ? qt : t0) * H + (qvalid ? qh : g * kHpg)) *
                                     kHeadDim + 8 * j;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const half8_t*>(qrow + 32 * s);
  }

  auto lds16 = [](uint32_t addr) -> half8_t { return *(const lds_half8_t*)(uintptr_t)addr; };

  // S^T of the chunk whose K image sits in kv[KP] (KP = chunk parity)
  auto scores = [&](auto KP_T, f32x4 (&sacc)[4]) {
    constexpr int KP = decltype(KP_T)::value;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sacc[mt] = zero4();
    // (fences: the scheduler would hoist every fragment read; registers)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const half8_t af =
            lds16(koff[s & 3] + (KP * kHalf + 256 * (s >> 2) + mt * 16 * (kHeadDim * 2)));
        sacc[mt] = mfma16(af, qf[s], sacc[mt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Mask cells past each query's n_kv (only chunks that reach past the
  // block's first token need it).  Cell of (mt, i): 16 mt + 4 j + i.
  auto mask = [&](int c, f32x4 (&sacc)[4]) {
    const int cbase = c * kChunk;
    if (cbase + kChunk > nkv_min) {
      const int lim = nkv_q - cbase - 4 * j;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * mt + i >= lim) sacc[mt][i] = -INFINITY;
    }
  };

  // max over this query's cells of the chunk, in scaled log2 units
  auto chunk_max = [&](const f32x4 (&sacc)[4]) {
    float m[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      m[mt] = fmaxf(fmaxf(sacc[mt][0], sacc[mt][1]), fmaxf(sacc[mt][2], sacc[mt][3]));
    return lane_group_max(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]))) * kScoreScaleLog2;
  };

  // P = 2^(x - m) as fp16 B operands of the two 32-cell PV k-steps; adds
  // the fp32 exponentials to l.  Slot e of k-step kk is S^T tile 2 kk + e/4,
  // register e % 4.
  auto probs = [&](const f32x4 (&sacc)[4], float m, float& l, half8_t (&pb)[2]) {
    const float nm = -m;
    float ls[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(sacc[2 * kk + (e >> 2)][e & 3], kScoreScaleLog2, nm));
        pb[kk][e] = (_Float16)p[e];
      }
      ls[kk] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    l += ls[0] + ls[1];
  };

  // O^T += V^T P^T for the chunk whose V^T image sits in kv[2 + VP]
  auto pv = [&](auto VP_T, const half8_t (&pb)[2], f32x4 (&oacc)[16]) {
    constexpr int VP = decltype(VP_T)::value;
    // (fences every four fragments, as in scores)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const half8_t af = lds16(voff[kk] + (VP * kHalf + mt * 16 * (kChunk * 2)));
        oacc[mt] = mfma16(af, pb[kk], oacc[mt]);
        if ((mt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
  };

  // One pass over the block's chunks; returns true when the fast pass must
  // be redone exactly (SAFE = false only).  The fast pass finds K(cb) in
  // LDS and V(cb), K(cb + 1) requested.
  auto run = [&](auto SAFE_T) -> bool {
    constexpr bool SAFE = decltype(SAFE_T)::value;
    f32x4 oacc[16];
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) oacc[mt] = zero4();
    float m_ref = -INFINITY, l_run = 0.f;
    bool over = false;

    // Exact pass, chunk c (parity P), one step at a time: K(c + 1) and
    // V(c + 1) load while chunk c's scores, online softmax and PV run.
    auto step = [&](int c, auto P_T) {
      constexpr int P = decltype(P_T)::value;
      wait_vmcnt0();  // this wave's copies of K(c) and V(c) have landed
      wg_barrier();   // ... every wave's; and nobody reads chunk c - 1 any more
      if (c + 1 < ce) {
        copy_k(c + 1);
        copy_v(c + 1);
      }
      f32x4 s_cur[4];
      scores(std::integral_constant<int, P>{}, s_cur);
      mask(c, s_cur);
      const float cm = chunk_max(s_cur);
      // exact online softmax (this step serves the exact pass only)
      const float m_new = fmaxf(m_ref, cm);
      if (__builtin_amdgcn_ballot_w64(m_new > m_ref) != 0ull) {
        const float alpha = fast_exp2(m_ref - m_new);  // 0 while m_ref = -inf
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) oacc[mt] *= alpha;
        m_ref = m_new;
      }
      half8_t pb[2];
      probs(s_cur, m_ref, l_run, pb);
      pv(std::integral_constant<int, P>{}, pb, oacc);
    };
    // The same chunk for the fast pass, as an explicit schedule of stages
    // of four MFMAs: the operand fragments of stage i + kAhead are read
    // while stage i multiplies, the softmax exponentials of chunk c are spread
    // over the score stages, and scheduler fences keep that order.
    // Every chunk runs the same body, so the buffer parity is a run-time
    // offset; the last chunk (LAST) has no next chunk to score, and its score
    // stages only compute the exponentials.
    auto step_fast = [&](int c, f32x4 (&s_cur)[4], f32x4 (&s_nxt)[4], auto LAST_T) {
      constexpr bool LAST = decltype(LAST_T)::value;
      constexpr int kS = 8;            // score stages (k-steps of chunk c + 1)
      constexpr int kStages = kS + 8;  // then PV stages: k-step t / 4, m-tiles 4 (t % 4) ..
      constexpr int kAhead = 1;        // stages whose fragments are read ahead
      const uint32_t kpar = ((c + 1 - cb) & 1) * kHalf, vpar = ((c - cb) & 1) * kHalf;
      wait_vmcnt0();  // this wave's copies of K(c+1) and V(c) have landed
      wg_barrier();   // ... every wave's; and nobody reads K(c) or V(c-1) any more
      mask(c, s_cur);
      // the chunk's buffer bases; every fragment is then base + immediate
      uint32_t kb[4], vb[2];
#pragma unroll
      for (int x = 0; x < 4; ++x) kb[x] = koff[x] + kpar;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) vb[kk] = voff[kk] + vpar;
      half8_t fr[kAhead + 1][4];
      auto load = [&](auto I, half8_t (&dst)[4]) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < kS) {
          if constexpr (!LAST) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              dst[mt] = lds16(kb[i & 3] + (256 * (i >> 2) + mt * 16 * (kHeadDim * 2)));
          }
        } else {
          constexpr int t = i - kS;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            dst[m] = lds16(vb[t >> 2] + ((4 * (t & 3) + m) * 16 * (kChunk * 2)));
        }
      };
      if constexpr (!LAST) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) s_nxt[mt] = zero4();
      }
      static_for<kAhead>([&](auto I) { load(I, fr[decltype(I)::value]); });
      // the workgroup's first chunk holds a visible cell of every query:
      // the reference is finite
      if (c == cb) m_ref = chunk_max(s_cur);
      const float nm = -m_ref;
      half8_t pb[2];  // P in B-operand slot order: k-step kk, slot e
      // exponentials of slots 2 i and 2 i + 1 (slot q = 8 kk + e), rounded
      // to fp16 at once; l sums the fp32 values
      auto expo2 = [&](int i) {
        const int kk = i >> 2, e = 2 * (i & 3);
        const float p0 =
            fast_exp2(__builtin_fmaf(s_cur[2 * kk + (e >> 2)][e & 3], kScoreScaleLog2, nm));
        const float p1 =
            fast_exp2(__builtin_fmaf(s_cur[2 * kk + (e >> 2)][(e & 3) + 1], kScoreScaleLog2, nm));
        pb[kk][e] = (_Float16)p0;
        pb[kk][e + 1] = (_Float16)p1;
        l_run += p0 + p1;
      };
      __builtin_amdgcn_sched_barrier(0);
      static_for<kStages>([&](auto I) {
        constexpr int i = decltype(I)::value;
        // the next images stream in from inside the stage sequence, not all
        // at the step's start: the LDS writes of the copies then interleave
        // with the fragment reads instead of meeting them in one burst.
        // 8 waves: K(c+2) after two score stages, V(c+1) after six; 4 waves
        // (twice the copies per wave): each image in halves, K after stages
        // 1 and 3, V after 5 and 7.
        if constexpr (kWaves == 8) {
          if constexpr (i == 2) {
            if (c + 2 < ce) copy_k(c + 2);
          }
          if constexpr (i == 6) {
            if (c + 1 < ce) copy_v(c + 1);
          }
        } else if constexpr (i == 1 || i == 3 || i == 5 || i == 7) {
          constexpr int h = (i == 1 || i == 5) ? 0 : 1;  // first or second half
          constexpr bool isk = i < 4;
          const int cc = isk ? c + 2 : c + 1;
          if (cc < ce) {
            const uint8_t* src = img_g + (int64_t)cc * kImg + (isk ? 0 : kHalf);
            const uint32_t dst =
                lds_addr(kv) + ((isk ? 0 : 2) + ((cc - cb) & 1)) * kHalf + w * (kHalf / kWaves);
#pragma unroll
            for (int op = (kCopyOps / 2) * h; op < (kCopyOps / 2) * (h + 1); ++op)
              copy16_to_lds(src, copy_voff[op], dst + 1024 * op);
          }
        }
        if constexpr (i + kAhead < kStages)
          load(std::integral_constant<int, i + kAhead>{}, fr[(i + kAhead) % (kAhead + 1)]);
        if constexpr (i < kS) {
          if constexpr (!LAST) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              s_nxt[mt] = mfma16(fr[i % (kAhead + 1)][mt], qf[i], s_nxt[mt]);
          }
          expo2(i);
          if constexpr (!LAST && i + kAhead < kStages) {
            // inside the stage: one product, one fragment read for the next
            // stage, one VALU op (the exponentials), four times over
            static_for<4>([&](auto) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
              __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
            });
          }
        } else {
          constexpr int t = i - kS;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            oacc[4 * (t & 3) + m] =
                mfma16(fr[i % (kAhead + 1)][m], pb[t >> 2], oacc[4 * (t & 3) + m]);
          if constexpr (kWaves == 4 && i + kAhead < kStages) {
            // one wave per SIMD: alternate products and the next stage's
            // fragment reads (with two waves per SIMD the other wave fills
            // the gaps, and the scheduler's own order is as fast)
            static_for<4>([&](auto) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            });
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    if constexpr (SAFE) {
      copy_k(cb);
      copy_v(cb);
      int c = cb;
      for (; c + 1 < ce; c += 2) {
        step(c, P0{});
        step(c + 1, P1{});
      }
      if (c < ce) step(c, P0{});
    } else {
      f32x4 s_cur[4];
      scores(std::integral_constant<int, 0>{}, s_cur);
      // two chunks per trip: the score registers trade roles, no copies
      f32x4 s_alt[4];
      int c = cb;
      for (; c + 2 < ce; c += 2) {
        step_fast(c, s_cur, s_alt, F_{});
        step_fast(c + 1, s_alt, s_cur, F_{});
      }
      if (c + 1 < ce) {
        step_fast(c, s_cur, s_alt, F_{});
        step_fast(c + 1, s_alt, s_cur, T_{});
      } else {
        step_fast(c, s_cur, s_alt, T_{});
      }
    }

    // ---- finalise: O / l -> fp16; lane (n, j) holds dims 16 mt + 4 j + i
    float l_tot = lane_group_sum(l_run);
    if constexpr (!SAFE) {
      // workgroup vote: every P value is below l, so l < 65504 means no P
      // overflowed fp16; otherwise (scores far above the reference of the
      // workgroup's first chunk) its chunks are redone exactly
      over = qvalid && !(l_tot < kP16Max);
      if (__builtin_amdgcn_ballot_w64(over) != 0ull) s_redo = 1;
      __syncthreads();
      if (s_redo) return true;
    }

    // ---- a split block's pieces: each publishes its partial (O, m, l) and
    // counts itself; the one counted last merges every piece's partial and
    // writes the block.  Partials travel with write-through stores and loads
    // that read past this XCD's L2 (cache policy sc1: agent scope), so no
    // cache write-back or invalidation is needed around the count: a
    // piece's stores complete (vmcnt) before a barrier, then one relaxed
    // agent-scope add.  No piece ever waits for another.  The merge runs in
    // piece order whichever piece merges, so the result does not depend on
    // the order of arrival.
    if constexpr (kSplit) {
      if (sb >= 0) {
        constexpr int kSc1 = 16;  // cache policy bit sc1
        constexpr int kPart = part_floats(kWaves);
        const int np = sp.pieces;
        auto rsrc = [&](int p) {
          return __builtin_amdgcn_make_buffer_rsrc(sp.part + ((int64_t)sb * np + p) * kPart,
                                                   (short)0, 4 * kPart, kBufferFlags);
        };
        const auto rs_own = rsrc(piece);
        const int o_off = w * (16 * 64 * 16) + 16 * lane;  // + 1024 mt: (w, mt, lane) group
        const int ml_off = (kQpb * kHeadDim + 2 * (kQpw * w + n)) * 4;
        int* cntp = sp.cnt + sb;
#pragma unroll
        for (int mt = 0; mt < 16; ++mt)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, oacc[mt]), rs_own,
                                                 o_off + 1024 * mt, 0, kSc1);
        if (j == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_ref), rs_own, ml_off, 0, kSc1);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_tot), rs_own, ml_off + 4, 0,
                                                kSc1);
        }
        wait_vmcnt0();    // this thread's partial has reached memory ...
        __syncthreads();  // ... and every thread's, before the count
        if (tid == 0)
          s_flag = __hip_atomic_fetch_add(cntp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_flag != np - 1) return false;  // a piece counted later merges
        // every other piece's partial is complete: log-sum-exp merge in
        // piece order, this piece's from its registers
        float mp[kMaxPieces], lp[kMaxPieces], mm = -INFINITY;
#pragma unroll
        for (int p = 0; p < kMaxPieces; ++p) {
          if (p < np) {
            const auto rs = rsrc(p);
            mp[p] = p == piece ? m_ref
                               : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ml_off, 0, kSc1));
            lp[p] = p == piece ? l_tot
                               : __uint_as_float(
                                     __builtin_amdgcn_raw_buffer_load_b32(rs, ml_off + 4, 0, kSc1));
            mm = fmaxf(mm, mp[p]);
          }
        }
        f32x4 acc[16];
        float lsum = 0.f;
#pragma unroll
        for (int p = 0; p < kMaxPieces; ++p) {
          if (p < np) {
            const float wp = fast_exp2(mp[p] - mm);
            lsum = p == 0 ? wp * lp[p] : lsum + wp * lp[p];
            const auto rs = rsrc(p);
#pragma unroll
            for (int mt = 0; mt < 16; ++mt) {
              const f32x4 op =
                  p == piece ? oacc[mt]
                             : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             rs, o_off + 1024 * mt, 0, kSc1));
              acc[mt] = p == 0 ? wp * op : acc[mt] + wp * op;
            }
          }
        }
        l_tot = lsum;
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) oacc[mt] = acc[mt];
        if (tid == 0) __hip_atomic_store(cntp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    if constexpr (SAFE) {
      if (qvalid) {
        const float inv = 1.f / l_tot;
        _Float16* orow = a.out + ((int64_t)qt * H + qh) * kHeadDim + 4 * j;
#pragma unroll
        for (int mt = 0; mt < 16; ++mt) {
          half4_t o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = (_Float16)(oacc[mt][i] * inv);
          *reinterpret_cast<half4_t*>(orow + 16 * mt) = o;
        }
      }
    } else {
      // O^T goes through LDS (the chunk buffers: every wave is past the
      // vote's barrier, so none reads them any more) and leaves as 16-byte
      // stores, two whole output rows per store instruction.  The stores are
      // non-temporal: nothing in this kernel reads O, and so marked the 24 MB
      // of output at T=1984 cost the launch ~3% less time and ~1 MB less of
      // chunk images fetched again
      constexpr int kRowB = kHeadDim * 2 + 16;  // padded row: spreads the banks
      uint8_t* tile = kv + w * (kQpw * kRowB);
      const float inv = qvalid ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        half4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (_Float16)(oacc[mt][i] * inv);
        *reinterpret_cast<half4_t*>(tile + n * kRowB + 2 * (16 * mt + 4 * j)) = o;
      }
      const int half_row = lane >> 5, seg = lane & 31;
#pragma unroll
      for (int r = 0; r < kQpw / 2; ++r) {
        const int qn = 2 * r + half_row;  // query slot kQpw w + qn
        const int s2 = q0 + kQpw * w + qn;
        const half8_t v = *reinterpret_cast<const half8_t*>(tile + qn * kRowB + 16 * seg);
        if (s2 <= q_last)
          __builtin_nontemporal_store(
              v, reinterpret_cast<half8_t*>(a.out + ((int64_t)(s2 / kHpg) * H + g * kHpg +
                                                     s2 % kHpg) * kHeadDim + 8 * seg));
      }
    }
    return false;
  };

  // Q and every wave's share of K(0) are in before V(0) and K(1) are
  // requested: a compiler-visible wait, so that no count-based wait for the
  // Q loads is left inside the loop (it would also wait for the copies,
  // which the compiler does not count), then a barrier
  if (tid == 0) s_redo = 0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  copy_v(cb);
  if (cb + 1 < ce) copy_k(cb + 1);
  if (run(std::false_type{})) run(std::true_type{});
}

namespace {

// Bytes of the dequantised chunk images: cells [0, pos0 + t_count) of every
// group, 64 KB per (group, 64-cell chunk).
int64_t tile_image_bytes(int G, int t_count, int pos0) {
  if (t_count <= 0) return 0;
  const int64_t n_needed = (int64_t)pos0 + t_count;  // cells the last identity token sees
  const int64_t nchunks = (n_needed + kChunk - 1) / kChunk;
  return (int64_t)G * nchunks * kImg;
}
// Bytes of the split pieces' counters (256-byte rounded) and partials on
// the 4-wave grid.
int64_t split_bytes(int G, int n_split, int pieces) {
  if (n_split <= 0) return 0;
  const int64_t n = (int64_t)G * n_split;
  return (n * 4 + 255) / 256 * 256 + pieces * n * (int64_t)part_floats(4) * 4;
}

// Which blocks of a launch run as several pieces.  Only a 4-wave grid that
// leaves CUs idle splits, and only into those idle CUs, so every workgroup
// still starts in the launch's first round (a second round starts late on
// this hardware).  A piece's publish, count and the last piece's merge cost
// about three chunk times, so only blocks of at least 12 chunks (and 3/4
// of the longest block's) are split: the long blocks of a few tokens after
// a long prefix.  They get as many pieces (up to 3, each at least 6
// chunks) as the idle CUs allow for all of them; when even 2 pieces each do
// not fit, nothing is split (an unsplit long block would still set the
// launch's length).
struct SplitPlan {
  int n_split = 0, pieces = 1;
};
SplitPlan split_plan(int G, int t_count, int pos0) {
  SplitPlan sp;
  if (t_count <= 0 || tile_blocks(t_count, 8) * G >= kCus) return sp;
  const int nb = tile_blocks(t_count, 4);
  const int idle = kCus - nb * G;
  const int top = block_chunks(nb - 1, t_count, pos0, 4);
  if (idle < G || top < 12) return sp;
  const int lim = max(12, (3 * top + 3) / 4);
  int count = 0;
  while (count < nb && block_chunks(nb - 1 - count, t_count, pos0, 4) >= lim) ++count;
  // every token of a split block must see a cell of each piece's first
  // chunk: 64 cb < pos0 + t0 + 1 for the block's first token t0
  auto fits = [&](int s, int k) {
    for (int b = nb - s; b < nb; ++b) {
      const int nch = block_chunks(b, t_count, pos0, 4);
      const int64_t t0 = (int64_t)b * tile_queries(4) / kHpg;
      if ((int64_t)kChunk * piece_start(nch, k - 1, k) >= pos0 + t0 + 1) return false;
    }
    return true;
  };
  for (int k = kMaxPieces; k >= 2; --k) {
    if (lim >= 6 * k && count * (k - 1) * G <= idle && fits(count, k)) {
      sp.n_split = count;
      sp.pieces = k;
      return sp;
    }
  }
  return sp;
}
// The plan and its pointers, or no split when ws_bytes does not hold the
// plan's pieces beyond the images (a part of the plan would leave long
// blocks whole, and they would still set the launch's length).
TileSplit split_args(int G, int t_count, int pos0, void* ws, int64_t ws_bytes) {
  const SplitPlan plan = split_plan(G, t_count, pos0);
  const int64_t room = ws_bytes - tile_image_bytes(G, t_count, pos0);
  const int s = split_bytes(G, plan.n_split, plan.pieces) <= room ? plan.n_split : 0;
  TileSplit sp{s, s > 0 ? plan.pieces : 1, nullptr, nullptr};
  if (s > 0) {
    uint8_t* base = static_cast<uint8_t*>(ws) + tile_image_bytes(G, t_count, pos0);
    const int64_t n = (int64_t)G * s;
    sp.cnt = reinterpret_cast<int*>(base);
    sp.part = reinterpret_cast<float*>(base + (n * 4 + 255) / 256 * 256);
  }
  return sp;
}

}  // namespace

int64_t tile_workspace_min_bytes(int G, int t_count, int pos0) {
  return tile_image_bytes(G, t_count, pos0);
}

int64_t tile_workspace_bytes(int G, int t_count, int pos0) {
  const SplitPlan plan = split_plan(G, t_count, pos0);
  return tile_image_bytes(G, t_count, pos0) + split_bytes(G, plan.n_split, plan.pieces);
}

hipError_t launch_tile_prepare(const RowArgs& a, int t_count, void* ws, int64_t ws_bytes,
                               hipStream_t stream) {
  if (t_count <= 0) return hipSuccess;
  const int n_needed = a.pos0 + t_count;
  const int nchunks = (n_needed + kChunk - 1) / kChunk;
  const TileSplit sp = split_args(a.G, t_count, a.pos0, ws, ws_bytes);
  dequant_chunks_kernel<<<dim3((2 * a.G * nchunks + 7) / 8 * 32), dim3(64), 0, stream>>>(
      a, n_needed, nchunks, static_cast<uint8_t*>(ws), sp.cnt, a.G * sp.n_split);
  return hipGetLastError();
}

hipError_t launch_tile_attend(const RowArgs& a, int t_count, void* ws, int64_t ws_bytes,
                              hipStream_t stream) {
  if (t_count <= 0) return hipSuccess;
  const int n_needed = a.pos0 + t_count;
  const int nchunks = (n_needed + kChunk - 1) / kChunk;
  const uint8_t* img = static_cast<const uint8_t*>(ws);
  const int blocks8 = tile_blocks(t_count, 8);
  if (blocks8 * a.G >= kCus) {
    flash_tile_kernel<8, false><<<dim3(blocks8 * a.G), dim3(8 * 64), 0, stream>>>(
        a, t_count, nchunks, img, TileSplit{0, 1, nullptr, nullptr});
  } else {
    const int blocks4 = tile_blocks(t_count, 4);
    const TileSplit sp = split_args(a.G, t_count, a.pos0, ws, ws_bytes);
    const dim3 grid((blocks4 + (sp.pieces - 1) * sp.n_split) * a.G);
    if (sp.n_split > 0)
      flash_tile_kernel<4, true><<<grid, dim3(4 * 64), 0, stream>>>(a, t_count, nchunks, img, sp);
    else
      flash_tile_kernel<4, false><<<grid, dim3(4 * 64), 0, stream>>>(a, t_count, nchunks, img, sp);
  }
  return hipGetLastError();
}

}  // namespace qsa
