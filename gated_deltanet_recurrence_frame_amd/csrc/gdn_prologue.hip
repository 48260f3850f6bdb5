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
// One thread per gate; a row of d io elements takes one 16-byte piece per
// lane on 16 lanes (a DPP row; 32 lanes for fp32 rows of more than 16
// pieces), so a wave reads whole rows contiguously and the row's sums
// come from a cross-lane reduction.
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

// Sum over the LPR lanes of a row (a DPP row, or two adjacent ones).
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  v = row_sum16(v);
  if constexpr (LPR == 32) v += __shfl_xor(v, 16);
  return v;
}

template <int IO, int LPR>
__global__ __launch_bounds__(kPrologueThreads) void rows_normalize_kernel(const void* x, void* y,
                                                                         float* inv_out,
                                                                         int64_t rows, int ph) {
  const int64_t r = (int64_t)blockIdx.x * (kPrologueThreads / LPR) + threadIdx.x / LPR;
  const int pc = threadIdx.x % LPR;
  const bool live = r < rows && pc < ph;
  // every lane takes part in the row sums: no early return
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (live) v = reinterpret_cast<const u32x4*>(x)[r * ph + pc];
  const float ss = row_sum<LPR>(piece_sumsq<IO>(v));
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  if (live && y) reinterpret_cast<u32x4*>(y)[r * ph + pc] = piece_scale<IO>(v, inv);
  if (inv_out && r < rows && pc == 0) inv_out[r] = inv;
}

template <int IO, int LPR>
__global__ __launch_bounds__(kPrologueThreads) void rows_normalize_bwd_kernel(const void* x,
                                                                             void* g,
                                                                             int64_t rows, int ph) {
  typedef Piece<IO> P;
  const int64_t r = (int64_t)blockIdx.x * (kPrologueThreads / LPR) + threadIdx.x / LPR;
  const int pc = threadIdx.x % LPR;
  const bool live = r < rows && pc < ph;
  u32x4 xv = u32x4{0u, 0u, 0u, 0u}, gv = xv;
  if (live) {
    xv = reinterpret_cast<const u32x4*>(x)[r * ph + pc];
    gv = reinterpret_cast<const u32x4*>(g)[r * ph + pc];
  }
  float f[P::n], h[P::n];
  P::get(xv, f);
  P::get(gv, h);
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int e = 0; e < P::n; ++e) {
    ss = fmaf(f[e], f[e], ss);
    dot = fmaf(f[e], h[e], dot);
  }
  ss = row_sum<LPR>(ss);
  dot = row_sum<LPR>(dot);
  // dx = (g - x^ (x^ . g)) / |x| = g inv - x (x . g) inv^3
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  const float c = dot * inv * inv;
#pragma unroll
  for (int e = 0; e < P::n; ++e) h[e] = (h[e] - f[e] * c) * inv;
  if (live) reinterpret_cast<u32x4*>(g)[r * ph + pc] = P::put(h);
}

static dim3 grid_for(int64_t n) {
  return dim3((unsigned)((n + kPrologueThreads - 1) / kPrologueThreads));
}
// rows of ph pieces, LPR lanes a row
static dim3 grid_rows(int64_t rows, int lpr) {
  const int64_t per = kPrologueThreads / lpr;
  return dim3((unsigned)((rows + per - 1) / per));
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

hipError_t launch_rows_normalize(const void* x, void* y, float* inv, int64_t rows, int d, int io,
                                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int ph = d * (io == IO_BF16 ? 2 : 4) / 16;
  if (d % 16 != 0 || ph > (io == IO_BF16 ? 16 : 32)) return hipErrorInvalidValue;
  const dim3 blk(kPrologueThreads);
  if (io == IO_BF16)
    hipLaunchKernelGGL((rows_normalize_kernel<IO_BF16, 16>), grid_rows(rows, 16), blk, 0, s, x, y,
                       inv, rows, ph);
  else if (ph <= 16)
    hipLaunchKernelGGL((rows_normalize_kernel<IO_F32, 16>), grid_rows(rows, 16), blk, 0, s, x, y,
                       inv, rows, ph);
  else
    hipLaunchKernelGGL((rows_normalize_kernel<IO_F32, 32>), grid_rows(rows, 32), blk, 0, s, x, y,
                       inv, rows, ph);
  return hipGetLastError();
}

hipError_t launch_rows_normalize_bwd(const void* x, void* g, int64_t rows, int d, int io,
                                     hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int ph = d * (io == IO_BF16 ? 2 : 4) / 16;
  if (d % 16 != 0 || ph > (io == IO_BF16 ? 16 : 32)) return hipErrorInvalidValue;
  const dim3 blk(kPrologueThreads);
  if (io == IO_BF16)
    hipLaunchKernelGGL((rows_normalize_bwd_kernel<IO_BF16, 16>), grid_rows(rows, 16), blk, 0, s,
                       x, g, rows, ph);
  else if (ph <= 16)
    hipLaunchKernelGGL((rows_normalize_bwd_kernel<IO_F32, 16>), grid_rows(rows, 16), blk, 0, s,
                       x, g, rows, ph);
  else
    hipLaunchKernelGGL((rows_normalize_bwd_kernel<IO_F32, 32>), grid_rows(rows, 32), blk, 0, s,
                       x, g, rows, ph);
  return hipGetLastError();
}

}  // namespace gdn
