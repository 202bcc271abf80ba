// qsa_merge.hip -- log-sum-exp merge of split-mode chunk partials.
//
// Pages: "round 27 track b - qsa prep and merge" (decision; correctness:
// partial records of 258 floats per head, 24*258 per chunk, (m, l) after the
// 256 output dims).  For token t and head h, with nk = ceil(n_sel(t)/64)
// records (o_k, m_k, l_k):
//   M = max_k m_k,  L = sum_k l_k e^(m_k - M),  out = sum_k e^(m_k - M) o_k / L.
//
// One wavefront per (token, head).  Lanes first read the (m, l) pairs of
// different chunks in parallel (maxima and sums reduced across the wave),
// then every lane streams its 4 output dims over the chunks.  Records are
// 1032 bytes apart, so the loads are 8-byte (float2) accesses.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                    _Float16* __restrict__ out, int T, int H,
                                                    int pos0, int budget, int KC) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= T * H) return;
  const int t = pair / H, h = pair % H;
  const int64_t nkv = (int64_t)pos0 + t + 1;
  const int nsel = nkv < budget ? (int)nkv : budget;
  const int nk = (nsel + kChunk - 1) / kChunk;
  const float* base = part + ((int64_t)t * KC * H + h) * kRec;
  const int64_t kstride = (int64_t)H * kRec;

  // maxima and sums across chunks, lane-parallel
  float M = -INFINITY;
  for (int k = lane; k < nk; k += 64) M = fmaxf(M, base[k * kstride + kHeadDim]);
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
  for (int k = lane; k < nk; k += 64) {
    const float2 ml = *reinterpret_cast<const float2*>(base + k * kstride + kHeadDim);
    L += ml.y * expf(ml.x - M);
  }
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);

  float4 acc = {0.f, 0.f, 0.f, 0.f};
  const int d0 = lane * 4;
  for (int k = 0; k < nk; ++k) {
    const float* rec = base + k * kstride;
    const float w = expf(rec[kHeadDim] - M);
    const float2 a = *reinterpret_cast<const float2*>(rec + d0);
    const float2 b = *reinterpret_cast<const float2*>(rec + d0 + 2);
    acc.x += w * a.x;
    acc.y += w * a.y;
    acc.z += w * b.x;
    acc.w += w * b.y;
  }
  const float inv = 1.f / L;
  half4_t o;
  o[0] = (_Float16)(acc.x * inv);
  o[1] = (_Float16)(acc.y * inv);
  o[2] = (_Float16)(acc.z * inv);
  o[3] = (_Float16)(acc.w * inv);
  *reinterpret_cast<half4_t*>(out + ((int64_t)t * H + h) * kHeadDim + d0) = o;
}

hipError_t launch_merge(const float* part, _Float16* out, int T, int H, int pos0, int budget,
                        hipStream_t stream) {
  const int KC = (budget + kChunk - 1) / kChunk;
  const int pairs = T * H;
  dim3 grid((pairs + 3) / 4), block(256);
  merge_kernel<<<grid, block, 0, stream>>>(part, out, T, H, pos0, budget, KC);
  return hipGetLastError();
}

}  // namespace qsa
