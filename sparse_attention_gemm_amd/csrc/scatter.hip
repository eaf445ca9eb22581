// scatter.hip -- the selection inverted: per latent row (or indexer key), the
// (query, entry) pairs that selected it, and a deterministic sum of per-pair
// vectors into each row.
//
// The backward passes produce one gradient vector per selected pair (query t,
// entry a of idx[t]) and need, for every row r, the sum over the pairs whose
// entry is r -- a scatter-add over the top-k output.  Instead of
// floating-point atomics (whose summation order, and so whose rounding,
// changes from run to run), the selection of a chunk of Tc queries is
// inverted with a counting sort:
//   1. cnt[r]  = number of pairs with entry r          (integer atomics: exact)
//   2. start   = exclusive prefix sum of cnt           (one workgroup)
//   3. list[start[r] + i] = pair index of r's i-th pair (in arrival order)
// and the reduce sorts each row's list by pair index before it sums, so every
// row is summed in increasing (query, entry) order, whatever the arrival
// order was.  Rows with more pairs than the sort holds in LDS are summed in
// arrival order (only possible when a query lists one row several times).
#include "dsa_common.h"
#include "dsa_launch.h"

namespace {

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float *__restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// pairs of a chunk: pair p = t * k + a for t < Tc; its entry idx[p], valid in [0, N)
__global__ __launch_bounds__(256) void scatter_count_kernel(const int32_t *__restrict__ idx, int64_t npairs,
                                                            int64_t N, int32_t *__restrict__ cnt) {
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < npairs; p += (int64_t)gridDim.x * 256) {
    const int32_t r = idx[p];
    if (r >= 0 && r < N) atomicAdd(cnt + r, 1);
  }
}

// start[0..N] = exclusive prefix sum of cnt[0..N); one workgroup of 1024
// threads over pages of 16384 entries.  Thread t owns the 16 consecutive
// entries 16 t .. 16 t + 15 of a page: it loads them as four 16-byte vectors
// (scalar loads only in a ragged last page), scans them in registers, and a
// wave scan plus one cross-wave step give every run its offset.  (Scalar
// accesses throughout if cnt or start is not 16-byte aligned.)
__global__ __launch_bounds__(1024) void scatter_scan_kernel(const int32_t *__restrict__ cnt, int64_t N,
                                                            int32_t *__restrict__ start) {
  constexpr int kRun = 16;
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool vec = ((reinterpret_cast<uintptr_t>(cnt) | reinterpret_cast<uintptr_t>(start)) & 15) == 0;
  int32_t carry = 0;  // total of the pages before this one
  for (int64_t p0 = 0; p0 < N; p0 += (int64_t)kRun * 1024) {
    const int64_t b = p0 + (int64_t)kRun * tid;
    const bool whole = vec && b + kRun <= N;
    int32_t v[kRun];
    if (whole) {
#pragma unroll
      for (int q = 0; q < kRun / 4; ++q) {
        const i32x4 x = *reinterpret_cast<const i32x4 *>(cnt + b + 4 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * q + j] = x[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRun; ++j) v[j] = b + j < N ? cnt[b + j] : 0;
    }
    int32_t inc[kRun];  // inclusive prefix within the run
    inc[0] = v[0];
#pragma unroll
    for (int j = 1; j < kRun; ++j) inc[j] = inc[j - 1] + v[j];
    const int32_t s = inc[kRun - 1];
    int32_t ws = s;  // inclusive scan of the run totals within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t x = __shfl_up(ws, o);
      if (lane >= o) ws += x;
    }
    if (lane == 63) wsum[wave] = ws;
    __syncthreads();
    int32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int32_t x = wsum[w];
      before += w < wave ? x : 0;
      total += x;
    }
    __syncthreads();  // wsum is rewritten for the next page
    const int32_t excl = carry + before + ws - s;  // entries before this run
    if (whole) {
#pragma unroll
      for (int q = 0; q < kRun / 4; ++q) {
        i32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = excl + inc[4 * q + j] - v[4 * q + j];
        *reinterpret_cast<i32x4 *>(start + b + 4 * q) = o;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRun; ++j)
        if (b + j < N) start[b + j] = excl + inc[j] - v[j];
    }
    carry += total;
  }
  if (tid == 0) start[N] = carry;
}

__global__ __launch_bounds__(256) void scatter_fill_kernel(const int32_t *__restrict__ idx, int64_t npairs, int64_t N,
                                                           const int32_t *__restrict__ start,
                                                           int32_t *__restrict__ cursor, int32_t *__restrict__ list) {
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < npairs; p += (int64_t)gridDim.x * 256) {
    const int32_t r = idx[p];
    if (r >= 0 && r < N) list[start[r] + atomicAdd(cursor + r, 1)] = (int32_t)p;
  }
}

constexpr int kSortCap = 4096;  // pairs of one row sorted in LDS

// Y[r, :] += sum over r's pairs p, in increasing p, of X[p, :].  One
// workgroup of BS threads per row, NCOL columns per thread (W <= BS NCOL).
template <int BS, int NCOL>
__global__ __launch_bounds__(BS) void scatter_add_kernel(const int32_t *__restrict__ start,
                                                         const int32_t *__restrict__ list, const float *__restrict__ X,
                                                         int W, float *__restrict__ Y) {
  __shared__ int32_t keys[kSortCap];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t b = start[r], n = start[r + 1] - b;
  if (n == 0) return;  // uniform
  const bool sorted = n <= kSortCap;
  if (sorted) {
    int m = 1;
    while (m < n) m <<= 1;
    for (int i = tid; i < m; i += BS) keys[i] = i < n ? list[b + i] : 0x7FFFFFFF;
    __syncthreads();
    // bitonic sort, ascending
    for (int size = 2; size <= m; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < (m >> 1); i += BS) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t x = keys[lo], y = keys[hi];
          if ((x > y) == up) {
            keys[lo] = y;
            keys[hi] = x;
          }
        }
        __syncthreads();
      }
    }
  }
  float acc[NCOL];
#pragma unroll
  for (int j = 0; j < NCOL; ++j) acc[j] = 0.0f;
  constexpr int kAhead = 8;  // pairs whose loads are in flight together; the adds stay in order
  for (int i0 = 0; i0 < n; i0 += kAhead) {
    float v[kAhead][NCOL];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int i = i0 + u;
      const int32_t p = i < n ? (sorted ? keys[i] : list[b + i]) : -1;
#pragma unroll
      for (int j = 0; j < NCOL; ++j) {
        const int d = tid + BS * j;
        v[u][j] = (p >= 0 && d < W) ? X[(int64_t)p * W + d] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
#pragma unroll
      for (int j = 0; j < NCOL; ++j) acc[j] += v[u][j];
  }
#pragma unroll
  for (int j = 0; j < NCOL; ++j) {
    const int d = tid + BS * j;
    if (d < W) Y[r * W + d] += acc[j];
  }
}

// The same for bf16 X (W even): thread u of a row owns the column pairs
// 2 (u + BS j), 2 (u + BS j) + 1 and adds them in fp32, in the same order.
template <int BS, int NPAIR>
__global__ __launch_bounds__(BS) void scatter_add_bf16_kernel(const int32_t *__restrict__ start,
                                                              const int32_t *__restrict__ list,
                                                              const __bf16 *__restrict__ X, int W,
                                                              float *__restrict__ Y) {
  __shared__ int32_t keys[kSortCap];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t b = start[r], n = start[r + 1] - b;
  if (n == 0) return;  // uniform
  const bool sorted = n <= kSortCap;
  if (sorted) {
    int m = 1;
    while (m < n) m <<= 1;
    for (int i = tid; i < m; i += BS) keys[i] = i < n ? list[b + i] : 0x7FFFFFFF;
    __syncthreads();
    for (int size = 2; size <= m; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < (m >> 1); i += BS) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t x = keys[lo], y = keys[hi];
          if ((x > y) == up) {
            keys[lo] = y;
            keys[hi] = x;
          }
        }
        __syncthreads();
      }
    }
  }
  const int W2 = W / 2;
  float acc[NPAIR][2];
#pragma unroll
  for (int j = 0; j < NPAIR; ++j) acc[j][0] = acc[j][1] = 0.0f;
  constexpr int kAhead = 8;
  for (int i0 = 0; i0 < n; i0 += kAhead) {
    bf16x2 v[kAhead][NPAIR];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int i = i0 + u;
      const int32_t p = i < n ? (sorted ? keys[i] : list[b + i]) : -1;
#pragma unroll
      for (int j = 0; j < NPAIR; ++j) {
        const int d2 = tid + BS * j;
        v[u][j] = (p >= 0 && d2 < W2) ? *reinterpret_cast<const bf16x2 *>(X + (int64_t)p * W + 2 * d2)
                                      : bf16x2{0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
#pragma unroll
      for (int j = 0; j < NPAIR; ++j) {
        acc[j][0] += (float)v[u][j][0];
        acc[j][1] += (float)v[u][j][1];
      }
  }
#pragma unroll
  for (int j = 0; j < NPAIR; ++j) {
    const int d2 = tid + BS * j;
    if (d2 < W2) {
      Y[r * W + 2 * d2] += acc[j][0];
      Y[r * W + 2 * d2 + 1] += acc[j][1];
    }
  }
}

int grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

namespace dsa {

hipError_t launch_fill_zero_f32(float *p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_scatter_build(const int32_t *idx, int64_t npairs, int64_t N, int32_t *cnt, int32_t *start,
                                int32_t *list, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(N)), dim3(256), 0, s, cnt, N, 0);
  if (npairs > 0)
    hipLaunchKernelGGL(scatter_count_kernel, dim3(grid_for(npairs)), dim3(256), 0, s, idx, npairs, N, cnt);
  hipLaunchKernelGGL(scatter_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, N, start);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(N)), dim3(256), 0, s, cnt, N, 0);
  if (npairs > 0)
    hipLaunchKernelGGL(scatter_fill_kernel, dim3(grid_for(npairs)), dim3(256), 0, s, idx, npairs, N, start, cnt,
                       list);
  return hipGetLastError();
}

hipError_t launch_scatter_add(const int32_t *start, const int32_t *list, int64_t N, const float *X, int32_t W, float *Y,
                              hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (W <= 128)  // one wave per row, two columns per lane
    hipLaunchKernelGGL((scatter_add_kernel<64, 2>), dim3((uint32_t)N), dim3(64), 0, s, start, list, X, W, Y);
  else if (W <= 768)
    hipLaunchKernelGGL((scatter_add_kernel<256, 3>), dim3((uint32_t)N), dim3(256), 0, s, start, list, X, W, Y);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_scatter_add_bf16(const int32_t *start, const int32_t *list, int64_t N, const void *X, int32_t W,
                                   float *Y, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (W % 2 != 0 || W > 768) return hipErrorInvalidValue;
  hipLaunchKernelGGL((scatter_add_bf16_kernel<128, 3>), dim3((uint32_t)N), dim3(128), 0, s, start, list,
                     (const __bf16 *)X, W, Y);
  return hipGetLastError();
}

}  // namespace dsa
