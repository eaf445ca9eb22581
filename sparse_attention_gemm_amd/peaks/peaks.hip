// peaks.hip -- measured peaks of the three rates the roofline of the DSA path
// is priced against: dense FP8 (E4M3) MFMA, dense bf16 MFMA and HBM read
// bandwidth.  Not part of the hot path: the benchmark reports every kernel's
// fraction of the datasheet peak and of these measured peaks side by side.
//
//  * MFMA loops: every wave issues independent accumulator chains of one
//    MFMA shape (32x32x64 E4M3; 32x32x16 bf16), with operands in registers,
//    so nothing but the matrix pipe limits the rate.  The chip may lower its
//    clock under this load, exactly as it does under the path's own kernels;
//    the measured rate includes that.
//  * HBM read: a grid-stride stream of 16-byte loads over a buffer far larger
//    than the 256 MB last-level cache, each thread keeping kLoads loads in
//    flight.
// Each kernel folds its results into a value that is stored only if it hits an
// impossible constant, so no work can be removed.
//
// Also here: one E4M3 16x16x128 MFMA per wave on given operands, to measure
// how the matrix core sums the 128 products of each dot product (the caller
// compares with exact sums).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kAcc32 = 4;   // independent accumulators per wave
constexpr int kLoads = 4;   // 16-byte loads in flight per thread

__global__ __launch_bounds__(256) void fp8_mfma_loop(int iters, float *sink) {
  const int l = threadIdx.x & 63;
  i32x8 a, b;
  // E4M3 bytes 0x38..0x3F: finite values in [1, 1.875]
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + 0x01010101 * ((l + i) & 7);
    b[i] = 0x38383838 + 0x01010101 * ((l * 3 + i) & 7);
  }
  f32x16 c[kAcc32];
#pragma unroll
  for (int j = 0; j < kAcc32; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc32; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc32; ++j) s += c[j][0] + c[j][7] + c[j][15];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

// Both loops use the 32x32 shapes: with several 16x16 accumulators the
// compiler may copy the loop-carried accumulators between AGPRs and VGPRs
// every iteration, and the loop then measures the copies, not the pipe.
__global__ __launch_bounds__(256) void bf16_mfma_loop(int iters, float *sink) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.125f * ((l + i) & 7));
    b[i] = (__bf16)(1.0f - 0.0625f * ((l * 3 + i) & 7));
  }
  f32x16 c[kAcc32];
#pragma unroll
  for (int j = 0; j < kAcc32; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc32; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc32; ++j) s += c[j][0] + c[j][7] + c[j][15];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void hbm_read_stream(const f32x4 *__restrict__ x, int64_t n16, float *sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (; i + (kLoads - 1) * stride < n16; i += kLoads * stride) {
    f32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc += v[u];
  }
  for (; i < n16; i += stride) acc += x[i];
  const float s = acc[0] + acc[1] + acc[2] + acc[3];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

// Streaming write of n16 16-byte vectors (grid-stride, one store per
// iteration per lane); `nt` sets the streaming cache policy on the stores.
template <bool NT>
__global__ __launch_bounds__(256) void hbm_write_stream(f32x4 *__restrict__ x, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const f32x4 v = {1.f, 2.f, 3.f, 4.f};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    if (NT)
      __builtin_nontemporal_store(v, x + i);
    else
      x[i] = v;
  }
}

// Trial t: D[t] = A[t] B[t]^T, A[t] and B[t] [16][128] E4M3 bytes (row j of
// B[t] is column j of the MFMA's B operand), D[t] [16][16] fp32, zero
// accumulator input.  One wave per trial.
__global__ __launch_bounds__(64) void fp8_mfma_dot(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
                                                  float *__restrict__ D) {
  const int l = threadIdx.x, g = l >> 4, c = l & 15;
  const size_t t = blockIdx.x;
  const i32x8 a = *reinterpret_cast<const i32x8 *>(A + (t * 16 + c) * 128 + 32 * g);
  const i32x8 b = *reinterpret_cast<const i32x8 *>(B + (t * 16 + c) * 128 + 32 * g);
  const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) D[(t * 16 + 4 * g + r) * 16 + c] = d[r];
}

}  // namespace

extern "C" {

// FLOP per wave-iteration of the MFMA loops (kAcc32 instructions).
int64_t dsa_peak_fp8_flop_per_wave_iter(void) { return (int64_t)kAcc32 * 32 * 32 * 64 * 2; }
int64_t dsa_peak_bf16_flop_per_wave_iter(void) { return (int64_t)kAcc32 * 32 * 32 * 16 * 2; }

// Launch `blocks` workgroups of four waves, each running `iters` iterations;
// sink holds at least `blocks` floats.  Returns the hipError_t of the launch.
int dsa_peak_fp8_mfma(int blocks, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(fp8_mfma_loop, dim3(blocks), dim3(256), 0, s, iters, sink);
  return (int)hipGetLastError();
}
int dsa_peak_bf16_mfma(int blocks, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(bf16_mfma_loop, dim3(blocks), dim3(256), 0, s, iters, sink);
  return (int)hipGetLastError();
}
// Read `bytes` (a multiple of 16, 16-byte aligned) of device memory at x.
int dsa_peak_hbm_read(const void *x, int64_t bytes, int blocks, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_stream, dim3(blocks), dim3(256), 0, s, (const f32x4 *)x, bytes / 16, sink);
  return (int)hipGetLastError();
}

// `trials` E4M3 16x16x128 MFMAs on device operands A, B ([trials][16][128]
// bytes each) into D ([trials][16][16] fp32).
int dsa_peak_fp8_mfma_dot(const void *A, const void *B, float *D, int trials, hipStream_t s) {
  if (trials <= 0) return 0;
  hipLaunchKernelGGL(fp8_mfma_dot, dim3(trials), dim3(64), 0, s, (const uint8_t *)A, (const uint8_t *)B, D);
  return (int)hipGetLastError();
}

// Write `bytes` (a multiple of 16) to x with 16-byte stores; nt != 0 marks them streaming.
int dsa_peak_hbm_write(void *x, int64_t bytes, int blocks, int nt, hipStream_t s) {
  if (nt)
    hipLaunchKernelGGL(hbm_write_stream<true>, dim3(blocks), dim3(256), 0, s, (f32x4 *)x, bytes / 16);
  else
    hipLaunchKernelGGL(hbm_write_stream<false>, dim3(blocks), dim3(256), 0, s, (f32x4 *)x, bytes / 16);
  return (int)hipGetLastError();
}
}
