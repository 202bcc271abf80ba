// qsa_quantize.hip -- the K/V quantiser that fills the int8 cache the
// attention path reads: fp16 rows of 256 dims -> int8 codes and one fp16
// scale per 64-dim block.
//
// Pages: "round 6 track b - qsa flash" (delivered change: int8 K/V codes
// with four fp16 scales per cell, one per 64 dims) and "round 27 track b -
// qsa prep and merge" (the prep step that writes the cache).  The pages do
// not give the rounding rule; this is the plain absmax one, per row and
// 64-dim block:
//   scale = fp16(amax / 127),  code = clamp(rint(x / scale), -127, 127),
// with every code 0 when the scale is 0.  Both divisions are IEEE fp32
// (correctly rounded), rint and the fp16 conversion round to nearest even,
// so the codes are a deterministic function of the fp16 input.
//
// Work mapping: 16 lanes per row, 16 dims per lane (two 16-byte loads, one
// 16-byte code store); a 64-dim block is 4 consecutive lanes, whose absmax
// takes two xor shuffles.  256 threads = 16 rows per workgroup.  The kernel
// streams 512 B in and 264 B out per row: HBM-bound.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

constexpr int kRowsPerWg = 16;

__global__ __launch_bounds__(256) void quantize_kernel(const _Float16* x, int8_t* codes,
                                                       _Float16* scales, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + (threadIdx.x >> 4);
  const int seg = threadIdx.x & 15;  // dims 16 seg .. 16 seg + 15, block seg / 4
  // every lane of a 16-lane row group shares `row`, so the shuffles below
  // only ever pair lanes that are all present or all gone
  if (row >= rows) return;
  const _Float16* xr = x + row * kHeadDim + 16 * seg;
  const half8_t h0 = *reinterpret_cast<const half8_t*>(xr);
  const half8_t h1 = *reinterpret_cast<const half8_t*>(xr + 8);
  float v[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = (float)h0[e];
    v[8 + e] = (float)h1[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const _Float16 sc = (_Float16)(amax / 127.0f);
  const float s = (float)sc;
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
  if (s > 0.f) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float c = fminf(fmaxf(rintf(v[e] / s), -127.f), 127.f);
      packed[e >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (e & 3));
    }
  }
  *reinterpret_cast<u32x4*>(codes + row * kHeadDim + 16 * seg) =
      u32x4{packed[0], packed[1], packed[2], packed[3]};
  if ((seg & 3) == 0) scales[row * kNBlk + (seg >> 2)] = sc;
}

}  // namespace

hipError_t launch_quantize(const _Float16* x, int8_t* codes, _Float16* scales, int64_t rows,
                           hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t wgs = (rows + kRowsPerWg - 1) / kRowsPerWg;
  quantize_kernel<<<dim3((unsigned)wgs), dim3(256), 0, stream>>>(x, codes, scales, rows);
  return hipGetLastError();
}

}  // namespace qsa
