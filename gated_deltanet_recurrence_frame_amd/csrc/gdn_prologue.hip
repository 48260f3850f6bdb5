// Prologue of the GDN block and its chain rule (summary page, 方法步骤详情
// module 2: the hats on Q^_t and K^_t, read as per-token normalisation; the
// gates gamma_t in (0, 1) and beta_t in (0, 1) taken as sigmoids of logits).
//
// The frame form's forward fuses the normalisation into its Gram/write and
// output kernels; these elementwise passes serve the rest: the gates from
// logits (tiny next to the token rows), and normalised copies of q and k
// for the token form and the backward, whose gradients then go through the
// chain rule here:
//   x^ = x / |x|:      dx = (dx^ - x^ (x^ . dx^)) / |x|   (0 for a zero row)
//   p = sigmoid(z):    dz = dp p (1 - p)
// One thread per gate or per row of d io elements (16-byte pieces, two
// passes: the sums, then the rewritten row, which the first pass left in
// cache).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kPrologueThreads = 256;

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + expf(-x)); }

__global__ __launch_bounds__(kPrologueThreads) void sigmoid_kernel(const float* x, float* y,
                                                                  int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kPrologueThreads + threadIdx.x;
  if (i < n) y[i] = sigmoidf(x[i]);
}

__global__ __launch_bounds__(kPrologueThreads) void sigmoid_bwd_kernel(const float* x, float* g,
                                                                      int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kPrologueThreads + threadIdx.x;
  if (i < n) {
    const float p = sigmoidf(x[i]);
    g[i] = g[i] * (p * (1.f - p));
  }
}

// Elements of a 16-byte piece as floats.
template <int IO> struct Piece;
template <> struct Piece<IO_BF16> {
  static constexpr int n = 8;
  __device__ static void get(const u32x4& v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(v[e] << 16);
      f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  __device__ static u32x4 put(const float* f) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)f32_to_bf16_bits(f[2 * e]) | ((uint32_t)f32_to_bf16_bits(f[2 * e + 1]) << 16);
    return v;
  }
};
template <> struct Piece<IO_F32> {
  static constexpr int n = 4;
  __device__ static void get(const u32x4& v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
  __device__ static u32x4 put(const float* f) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(f[e]);
    return v;
  }
};

template <int IO>
__global__ __launch_bounds__(kPrologueThreads) void rows_normalize_kernel(const void* x, void* y,
                                                                         int64_t rows, int d) {
  typedef Piece<IO> P;
  const int64_t r = (int64_t)blockIdx.x * kPrologueThreads + threadIdx.x;
  if (r >= rows) return;
  const int np = d / P::n;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x) + r * np;
  u32x4* yr = reinterpret_cast<u32x4*>(y) + r * np;
  float ss = 0.f;
  for (int p = 0; p < np; ++p) {
    float f[P::n];
    P::get(xr[p], f);
#pragma unroll
    for (int e = 0; e < P::n; ++e) ss = fmaf(f[e], f[e], ss);
  }
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  for (int p = 0; p < np; ++p) {
    float f[P::n];
    P::get(xr[p], f);
#pragma unroll
    for (int e = 0; e < P::n; ++e) f[e] *= inv;
    yr[p] = P::put(f);
  }
}

template <int IO>
__global__ __launch_bounds__(kPrologueThreads) void rows_normalize_bwd_kernel(const void* x,
                                                                             void* g,
                                                                             int64_t rows, int d) {
  typedef Piece<IO> P;
  const int64_t r = (int64_t)blockIdx.x * kPrologueThreads + threadIdx.x;
  if (r >= rows) return;
  const int np = d / P::n;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x) + r * np;
  u32x4* gr = reinterpret_cast<u32x4*>(g) + r * np;
  float ss = 0.f, dot = 0.f;
  for (int p = 0; p < np; ++p) {
    float f[P::n], h[P::n];
    P::get(xr[p], f);
    P::get(gr[p], h);
#pragma unroll
    for (int e = 0; e < P::n; ++e) {
      ss = fmaf(f[e], f[e], ss);
      dot = fmaf(f[e], h[e], dot);
    }
  }
  // dx = (g - x^ (x^ . g)) / |x| = g inv - x (x . g) inv^3
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  const float c = dot * inv * inv;
  for (int p = 0; p < np; ++p) {
    float f[P::n], h[P::n];
    P::get(xr[p], f);
    P::get(gr[p], h);
#pragma unroll
    for (int e = 0; e < P::n; ++e) h[e] = (h[e] - f[e] * c) * inv;
    gr[p] = P::put(h);
  }
}

static dim3 grid_for(int64_t n) {
  return dim3((unsigned)((n + kPrologueThreads - 1) / kPrologueThreads));
}

hipError_t launch_sigmoid(const float* x, float* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sigmoid_kernel, grid_for(n), dim3(kPrologueThreads), 0, s, x, y, n);
  return hipGetLastError();
}

hipError_t launch_sigmoid_bwd(const float* x, float* g, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sigmoid_bwd_kernel, grid_for(n), dim3(kPrologueThreads), 0, s, x, g, n);
  return hipGetLastError();
}

hipError_t launch_rows_normalize(const void* x, void* y, int64_t rows, int d, int io,
                                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 16 != 0) return hipErrorInvalidValue;
  if (io == IO_BF16)
    hipLaunchKernelGGL(rows_normalize_kernel<IO_BF16>, grid_for(rows), dim3(kPrologueThreads), 0,
                       s, x, y, rows, d);
  else
    hipLaunchKernelGGL(rows_normalize_kernel<IO_F32>, grid_for(rows), dim3(kPrologueThreads), 0,
                       s, x, y, rows, d);
  return hipGetLastError();
}

hipError_t launch_rows_normalize_bwd(const void* x, void* g, int64_t rows, int d, int io,
                                     hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 16 != 0) return hipErrorInvalidValue;
  if (io == IO_BF16)
    hipLaunchKernelGGL(rows_normalize_bwd_kernel<IO_BF16>, grid_for(rows), dim3(kPrologueThreads),
                       0, s, x, g, rows, d);
  else
    hipLaunchKernelGGL(rows_normalize_bwd_kernel<IO_F32>, grid_for(rows), dim3(kPrologueThreads),
                       0, s, x, g, rows, d);
  return hipGetLastError();
}

}  // namespace gdn
