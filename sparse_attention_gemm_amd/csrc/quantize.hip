// Per-token E4M3 quantisation of indexer operands.
//
// The indexer runs in FP8 (mizuki-eaf.pages.dev, "DeepSeek Sparse Attention" /
// "How it works"; m.digipub.cc, section 2).  Each row gets one fp32 scale,
// amax/448, so that its largest element lands on E4M3's largest finite value;
// the payload is the E4M3 rounding (nearest-even, saturating) of x/scale.
//
// One wavefront per row; the row is read twice (the second read hits L2/L1),
// so HBM traffic is 4 B in + 1 B out per element plus 4 B per row.
#include "dsa_launch.h"

namespace {

__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const float *__restrict__ x, int64_t rows,
                                                            int32_t cols, uint8_t *__restrict__ x8,
                                                            float *__restrict__ scale) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const float4 *xr = reinterpret_cast<const float4 *>(x + r * cols);
  const int n4 = cols >> 2;
  float amax = 0.0f;
  for (int i = lane; i < n4; i += 64) {
    float4 v = xr[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = wave_max(amax);
  float s = __fdiv_rn(amax, 448.0f);
  if (!(s > 0.0f)) s = 1.0f;
  if (lane == 0) scale[r] = s;
  uint32_t *out = reinterpret_cast<uint32_t *>(x8 + r * cols);
  for (int i = lane; i < n4; i += 64) {
    float4 v = xr[i];
    // fp32 quotient (correctly rounded), clamped to the finite E4M3 range,
    // then the hardware's round-to-nearest-even conversion.
    float a = fminf(fmaxf(__fdiv_rn(v.x, s), -448.0f), 448.0f);
    float b = fminf(fmaxf(__fdiv_rn(v.y, s), -448.0f), 448.0f);
    float c = fminf(fmaxf(__fdiv_rn(v.z, s), -448.0f), 448.0f);
    float d = fminf(fmaxf(__fdiv_rn(v.w, s), -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    out[i] = (uint32_t)w;
  }
}

}  // namespace

namespace dsa {
hipError_t launch_quantize(const float *x, int64_t rows, int32_t cols, uint8_t *x8, float *scale,
                           hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, x, rows, cols, x8,
                     scale);
  return hipGetLastError();
}
}  // namespace dsa
