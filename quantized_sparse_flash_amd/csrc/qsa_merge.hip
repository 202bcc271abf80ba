// qsa_merge.hip -- log-sum-exp merge of split-mode chunk partials.
//
// Pages: "round 27 track b - qsa prep and merge" (decision; correctness:
// partial records of 258 floats per head, 24*258 per chunk, (m, l) after the
// 256 output dims).  For token t and head h, with nk = ceil(n_sel(t)/64)
// records (o_k, m_k, l_k):
//   M = max_k m_k,  L = sum_k l_k e^(m_k - M),  out = sum_k e^(m_k - M) o_k / L.
//
// Records may also cover cpr consecutive chunks each (the row pieces of a
// fused call): nk = ceil(ceil(n_sel(t)/64) / cpr) records per token, KC
// record slots per token in the array.
//
// Two wavefronts per (token, head), one per 128-dim half.  A pass over up to
// 32 records issues all of its loads at once -- lane i reads record i's
// (m, l), every lane reads its two dims of every record -- so a merge costs
// one memory round trip per 32 records; passes combine by the same online
// rescaling.  Records are 1032 bytes apart (8-byte aligned only), so the
// loads are 8-byte (float2) accesses.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// Records per pass: a lane keeps kGroup records' two floats in registers,
// so a pass issues all of its loads before it needs any of them.
constexpr int kGroup = 32;

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                    _Float16* __restrict__ out, int T, int H,
                                                    int pos0, int budget, int KC, int cpr) {
  const int lane = threadIdx.x & 63;
  // wave-uniform: two waves per (token, head), one per 128-dim half
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (item >= 2 * T * H) return;
  const int pair = item >> 1, half = item & 1;
  const int t = pair / H, h = pair % H;
  const int64_t nkv = (int64_t)pos0 + t + 1;
  const int nsel = nkv < budget ? (int)nkv : budget;
  const int nk = ((nsel + kChunk - 1) / kChunk + cpr - 1) / cpr;
  const float* base = part + ((int64_t)t * KC * H + h) * kRec;
  const int64_t kstride = (int64_t)H * kRec;
  const int d0 = 128 * half + 2 * lane;  // this lane's two output dims

  // running (M, L, acc) over passes of kGroup records: lane i holds the
  // (m, l) of record k0 + i, every lane the two dims of every record
  float M = -INFINITY, L = 0.f;
  float2 acc = {0.f, 0.f};
  for (int k0 = 0; k0 < nk; k0 += kGroup) {
    const int cnt = nk - k0 < kGroup ? nk - k0 : kGroup;
    float2 ml = {-INFINITY, 0.f};
    if (lane < cnt) ml = *reinterpret_cast<const float2*>(base + (k0 + lane) * kstride + kHeadDim);
    float2 v[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      if (i < cnt) v[i] = *reinterpret_cast<const float2*>(base + (int64_t)(k0 + i) * kstride + d0);
    float gm = ml.x;
    for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
    const float m_new = fmaxf(M, gm);
    const float alpha = expf(M - m_new);  // 0 on the first pass (M = -inf)
    M = m_new;
    const float wl = lane < cnt ? expf(ml.x - M) : 0.f;
    float ls = ml.y * wl;
    for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
    L = L * alpha + ls;
    acc.x *= alpha;
    acc.y *= alpha;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (i < cnt) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
        acc.x += w * v[i].x;
        acc.y += w * v[i].y;
      }
    }
  }
  const float inv = 1.f / L;
  half2_t o;
  o[0] = (_Float16)(acc.x * inv);
  o[1] = (_Float16)(acc.y * inv);
  *reinterpret_cast<half2_t*>(out + ((int64_t)t * H + h) * kHeadDim + d0) = o;
}

hipError_t launch_merge(const float* part, _Float16* out, int T, int H, int pos0, int budget,
                        int cpr, hipStream_t stream) {
  if (cpr < 1) return hipErrorInvalidValue;
  const int KC = ((budget + kChunk - 1) / kChunk + cpr - 1) / cpr;
  const int waves = 2 * T * H;
  dim3 grid((waves + 3) / 4), block(256);
  merge_kernel<<<grid, block, 0, stream>>>(part, out, T, H, pos0, budget, KC, cpr);
  return hipGetLastError();
}

}  // namespace qsa
