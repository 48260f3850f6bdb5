// Per-frame token contraction ("Gram / write" pass) of the frame-wise GDN.
//
// For one (batch b, frame t, head h) the kernel computes, over the N tokens
// of the frame,
//     C_r = scale_r * X_r^T diag(w) Y        (D x D, fp32),  r < NR
// where X_r and Y are the frame's [N, D] token rows of [B, L, H, D] tensors.
//   forward:  X_0 = K, X_1 = V, Y = K, w = beta, scales s^2 and s, giving
//             A_t = K^_t beta_t K^_t^T and U_t = V_t beta_t K^_t^T
//             (summary page, 方法步骤详情 module 2: the delta-rule Gram and
//             the write term of M_t and U_t);
//   backward: X_0 = dO, Y = Q, w = 1, scale 1, giving dO_t Q^_t^T, the
//             frame's own contribution to dLoss/dS_t.
// All tokens of a frame read the same S_{t-1}, so there is no intra-frame
// triangular structure: the contraction is a dense D x N x D product.
//
// Outputs are stored in the intermediate type (bf16 for bf16 io, fp32 for
// fp32 io): A_t row-major, U_t and dO_t Q^_t^T in the MFMA tile layout that
// the scan consumes.
//
// Layout of the work: one workgroup (4 waves) per (b, t, h), XCD-aware
// ordering so heads of one frame run on one XCD, two workgroups per CU.
// Tokens stream through LDS in chunks of CT rows (natural [token][feature]
// layout, double-buffered), the next chunk in flight in registers.
// Both MFMA operands need a feature's values over consecutive tokens; they
// are read with the gfx950 transposing LDS read.  The weight w multiplies
// the X operand in fp32 before rounding to bf16.  Tail tokens of the last
// chunk re-read the frame's last row and get weight 0, so they add exactly 0.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT, int NR, bool Y_IS_X0>
struct GramCfg {
  static constexpr int D = 16 * NT;
  static constexpr int ES = Io<IO>::bytes;
  static constexpr int CT = (IO == IO_BF16) ? 64 : 32;     // tokens per chunk
  static constexpr int NMAT = NR + (Y_IS_X0 ? 0 : 1);       // matrices staged
  static constexpr int MAT_ELEMS = CT * D;
  static constexpr int PR = D * ES / 16;                    // 16-byte pieces per row
  static constexpr int PIECES = NMAT * CT * PR;
  static constexpr int PPT = (PIECES + 255) / 256;          // pieces per thread
  static constexpr int STAGE_BYTES = NMAT * MAT_ELEMS * ES + CT * 4;
  static constexpr int RT = (NR * NT + 3) / 4;              // row tiles per wave
};

template <int IO, int NT, int NR, bool Y_IS_X0>
__global__ __launch_bounds__(256, 2) void gram_kernel(GramArgs a) {
  typedef GramCfg<IO, NT, NR, Y_IS_X0> C;
  typedef typename Io<IO>::elem E;
  constexpr int D = C::D;
  constexpr int SMEM = (2 * C::STAGE_BYTES > D * D * C::ES) ? 2 * C::STAGE_BYTES : D * D * C::ES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int total = a.B * a.Tc * a.H * a.P;
  const int item = xcd_item(blockIdx.x, total);
  const int sp = item % a.P;                       // token split
  const int h = (item / a.P) % a.H;
  const int tl = (item / (a.P * a.H)) % a.Tc;
  const int t = a.t0 + tl;
  const int b = item / (a.P * a.H * a.Tc);
  const int N = a.N;
  const long L = (long)a.T * N;
  const long row0 = (long)b * L + (long)t * N;   // first token row of the frame

  const E* srcs[3] = {static_cast<const E*>(a.x0), static_cast<const E*>(NR == 2 ? a.x1 : a.y),
                      static_cast<const E*>(a.y)};
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int nchunks_all = (N + C::CT - 1) / C::CT;
  const int cps = (nchunks_all + a.P - 1) / a.P;  // chunks per split
  const int cbeg = sp * cps;
  const int nchunks = min(nchunks_all, cbeg + cps) - cbeg;   // may be <= 0

  // Register staging of the next chunk.  A chunk's weights are masked
  // here: 0 past the frame's last token (whose row is re-read), 1 when
  // there are no weights.
  struct Pre {
    u32x4 v[C::PPT];
    float w;
  };
  auto issue = [&](Pre& P, int c) {
    const int c0 = (cbeg + c) * C::CT;
#pragma unroll
    for (int j = 0; j < C::PPT; ++j) {
      const int p = tid + 256 * j;
      if (p < C::PIECES) {
        const int m = p / (C::CT * C::PR);
        const int r = p % (C::CT * C::PR);
        const int row = r / C::PR, pc = r % C::PR;
        int tok = c0 + row;
        if (tok >= N) tok = N - 1;
        P.v[j] = *reinterpret_cast<const u32x4*>(srcs[m] + ((row0 + tok) * a.H + h) * (long)D +
                                                 pc * (16 / C::ES));
      }
    }
    if (tid < C::CT) {
      const int tok = c0 + tid;
      P.w = tok < N ? (a.w ? a.w[(row0 + tok) * a.H + h] : 1.0f) : 0.0f;
    }
  };
  auto commit = [&](const Pre& P, int stage) {
    char* base = smem + stage * C::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < C::PPT; ++j) {
      const int p = tid + 256 * j;
      if (p < C::PIECES) *reinterpret_cast<u32x4*>(reinterpret_cast<E*>(base) + p * (16 / C::ES)) = P.v[j];
    }
    if (tid < C::CT) reinterpret_cast<float*>(base + C::NMAT * C::MAT_ELEMS * C::ES)[tid] = P.w;
  };

  f32x4 acc[C::RT][NT];
#pragma unroll
  for (int j = 0; j < C::RT; ++j)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[j][ct] = zero4();

  auto compute = [&](int stage) {
    const char* base = smem + stage * C::STAGE_BYTES;
    const E* xs = reinterpret_cast<const E*>(base);
    const E* ys = Y_IS_X0 ? xs : xs + (C::NMAT - 1) * C::MAT_ELEMS;
    const float* ws = reinterpret_cast<const float*>(base + C::NMAT * C::MAT_ELEMS * C::ES);
    if constexpr (IO == IO_BF16) {
#pragma unroll
      for (int kb = 0; kb < C::CT / 32; ++kb) {
        const int k0 = kb * 32;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(ws + k0 + 8 * g);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(ws + k0 + 8 * g + 4);
        bf16x8 bfr[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          bfr[ct] = lds_col_frag_bf16(reinterpret_cast<const uint16_t*>(ys), D, k0, ct * 16);
        bf16x8 afr[C::RT];
#pragma unroll
        for (int j = 0; j < C::RT; ++j) {
          const int rtg = wave + 4 * j;
          if (rtg < NR * NT) {
            const int m = rtg / NT, ft = rtg % NT;
            afr[j] = lds_col_frag_bf16(reinterpret_cast<const uint16_t*>(xs + m * C::MAT_ELEMS), D,
                                       k0, ft * 16);
          }
        }
#pragma unroll
        for (int j = 0; j < C::RT; ++j) {
          const int rtg = wave + 4 * j;
          if (rtg < NR * NT) {
            bf16x8 af = afr[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              af[e] = static_cast<__bf16>(static_cast<float>(af[e]) * w0[e]);
              af[4 + e] = static_cast<__bf16>(static_cast<float>(af[4 + e]) * w1[e]);
            }
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) acc[j][ct] = mfma_bf16(af, bfr[ct], acc[j][ct]);
          }
        }
      }
    } else {
#pragma unroll 2
      for (int kb = 0; kb < C::CT / 4; ++kb) {
        const int k = kb * 4 + g;
        const float wv = ws[k];
        float bfr[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) bfr[ct] = reinterpret_cast<const float*>(ys)[k * D + ct * 16 + li];
#pragma unroll
        for (int j = 0; j < C::RT; ++j) {
          const int rtg = wave + 4 * j;
          if (rtg < NR * NT) {
            const int m = rtg / NT, ft = rtg % NT;
            const float af =
                reinterpret_cast<const float*>(xs + m * C::MAT_ELEMS)[k * D + ft * 16 + li] * wv;
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) acc[j][ct] = mfma_f32(af, bfr[ct], acc[j][ct]);
          }
        }
      }
    }
  };

  // Pipeline: chunk c is computed from LDS stage c % 2 while chunk c + 1 is
  // in flight in registers; two workgroups per CU overlap each other's
  // waits.
  Pre P;
  if (nchunks > 0) {
    issue(P, 0);
    commit(P, 0);
  }
  block_sync();
  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) issue(P, c + 1);
    compute(c & 1);
    if (c + 1 < nchunks) commit(P, (c + 1) & 1);
    block_sync();
  }

  // Epilogue: C[m][n] lives in lane (g, n) register r with m = 4g + r.
  // Outputs are in the intermediate type (the io type).  The tiles layout
  // is written straight from the accumulators (4 contiguous values per
  // lane); a row-major output is staged through LDS (the chunk buffers are
  // free after the last barrier) and stored in 16-byte pieces.
  if (a.P > 1) {   // fp32 partial sums, tile layout
    const long pbase = ((((long)sp * a.B + b) * a.H + h) * a.Tc + tl) * NR * (long)(D * D);
#pragma unroll
    for (int j = 0; j < C::RT; ++j) {
      const int rtg = wave + 4 * j;
      if (rtg < NR * NT) {
        const int m = rtg / NT, ft = rtg % NT;
        const float sc = (m == 0 ? a.scale0 : a.scale1);
        float* out = a.part + pbase + m * (long)(D * D);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          *reinterpret_cast<f32x4*>(out + ((ft * NT + ct) * 64 + lane) * 4) = sc * acc[j][ct];
      }
    }
    return;
  }
  const long obase = (((long)b * a.H + h) * a.T + t) * (long)(D * D);
#pragma unroll
  for (int j = 0; j < C::RT; ++j) {
    const int rtg = wave + 4 * j;
    if (rtg < NR * NT) {
      const int m = rtg / NT, ft = rtg % NT;
      if ((m == 0 ? a.layout0 : a.layout1) == LAYOUT_TILES) {
        E* out = static_cast<E*>(m == 0 ? a.out0 : a.out1) + obase;
        const float sc = (m == 0 ? a.scale0 : a.scale1);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          E* dst = out + ((ft * NT + ct) * 64 + lane) * 4;
          const f32x4 v = sc * acc[j][ct];
          if constexpr (IO == IO_BF16) {
            u32x2 pk;
            pk[0] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
            pk[1] = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
            *reinterpret_cast<u32x2*>(dst) = pk;
          } else {
            *reinterpret_cast<f32x4*>(dst) = v;
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    if ((m == 0 ? a.layout0 : a.layout1) != LAYOUT_ROWMAJOR) continue;
    E* stage = reinterpret_cast<E*>(smem);
    const float sc = (m == 0 ? a.scale0 : a.scale1);
#pragma unroll
    for (int j = 0; j < C::RT; ++j) {
      const int rtg = wave + 4 * j;
      if (rtg < NR * NT && rtg / NT == m) {
        const int ft = rtg % NT;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = sc * acc[j][ct][r];
            E* dst = stage + (ft * 16 + 4 * g + r) * D + ct * 16 + li;
            if constexpr (IO == IO_BF16)
              *dst = f32_to_bf16_bits(v);
            else
              *dst = v;
          }
      }
    }
    block_sync();
    u32x4* out = reinterpret_cast<u32x4*>(static_cast<E*>(m == 0 ? a.out0 : a.out1) + obase);
    for (int idx = tid; idx < D * D * C::ES / 16; idx += 256)
      out[idx] = reinterpret_cast<const u32x4*>(stage)[idx];
    block_sync();
  }
}

// Sum of the P fp32 partials of one (b, t, h) frame and matrix r, in split
// order, written in the intermediate type and the output's layout.  One
// thread per 4 contiguous values of the tile layout.
template <int IO, int NT, int NR>
__global__ __launch_bounds__(256) void gram_reduce_kernel(GramArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr int D = 16 * NT;
  constexpr int Q = D * D / 4;                 // 4-value groups per matrix
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long nframes = (long)a.B * a.H * a.Tc;
  if (gid >= nframes * NR * Q) return;
  const int q = (int)(gid % Q);
  const int m = (int)((gid / Q) % NR);
  const long f = gid / ((long)Q * NR);          // (b, h, tl)
  const int tl = (int)(f % a.Tc);
  const long bh = f / a.Tc;
  f32x4 sum = zero4();
  for (int p = 0; p < a.P; ++p)
    sum += *reinterpret_cast<const f32x4*>(a.part + (((long)p * nframes + f) * NR + m) * (long)(D * D) +
                                           (long)q * 4);
  const int lane = q % 64, tile = q / 64;
  const int ft = tile / NT, ct = tile % NT, g = lane >> 4, li = lane & 15;
  E* out = static_cast<E*>(m == 0 ? a.out0 : a.out1) + (bh * a.T + a.t0 + tl) * (long)(D * D);
  if ((m == 0 ? a.layout0 : a.layout1) == LAYOUT_TILES) {
    E* dst = out + (long)q * 4;
    if constexpr (IO == IO_BF16) {
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(sum[0]) | ((uint32_t)f32_to_bf16_bits(sum[1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(sum[2]) | ((uint32_t)f32_to_bf16_bits(sum[3]) << 16);
      *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
      *reinterpret_cast<f32x4*>(dst) = sum;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      E* dst = out + (ft * 16 + 4 * g + r) * D + ct * 16 + li;
      if constexpr (IO == IO_BF16)
        *dst = f32_to_bf16_bits(sum[r]);
      else
        *dst = sum[r];
    }
  }
}

template <int IO, int NT>
static hipError_t launch_gram_reduce_nt(const GramArgs& a, int nr, hipStream_t s) {
  const long n = (long)a.B * a.H * a.Tc * nr * (16 * NT) * (16 * NT) / 4;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (nr == 2)
    hipLaunchKernelGGL((gram_reduce_kernel<IO, NT, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gram_reduce_kernel<IO, NT, 1>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_gram_reduce_io(const GramArgs& a, int nt, int nr, hipStream_t s) {
  switch (nt) {
    case 1: return launch_gram_reduce_nt<IO, 1>(a, nr, s);
    case 2: return launch_gram_reduce_nt<IO, 2>(a, nr, s);
    case 3: return launch_gram_reduce_nt<IO, 3>(a, nr, s);
    case 4: return launch_gram_reduce_nt<IO, 4>(a, nr, s);
    case 5: return launch_gram_reduce_nt<IO, 5>(a, nr, s);
    case 6: return launch_gram_reduce_nt<IO, 6>(a, nr, s);
    case 7: return launch_gram_reduce_nt<IO, 7>(a, nr, s);
    case 8: return launch_gram_reduce_nt<IO, 8>(a, nr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gram_reduce(const GramArgs& a, int io, int nt, int nr, hipStream_t s) {
  return io == IO_BF16 ? launch_gram_reduce_io<IO_BF16>(a, nt, nr, s)
                       : launch_gram_reduce_io<IO_F32>(a, nt, nr, s);
}

template <int IO, int NT>
static hipError_t launch_gram_nt(const GramArgs& a, int nr, hipStream_t s) {
  const dim3 grid(a.B * a.Tc * a.H * a.P), block(256);
  if (nr == 2)
    hipLaunchKernelGGL((gram_kernel<IO, NT, 2, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gram_kernel<IO, NT, 1, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_gram_io(const GramArgs& a, int nt, int nr, hipStream_t s) {
  switch (nt) {
    case 1: return launch_gram_nt<IO, 1>(a, nr, s);
    case 2: return launch_gram_nt<IO, 2>(a, nr, s);
    case 3: return launch_gram_nt<IO, 3>(a, nr, s);
    case 4: return launch_gram_nt<IO, 4>(a, nr, s);
    case 5: return launch_gram_nt<IO, 5>(a, nr, s);
    case 6: return launch_gram_nt<IO, 6>(a, nr, s);
    case 7: return launch_gram_nt<IO, 7>(a, nr, s);
    case 8: return launch_gram_nt<IO, 8>(a, nr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gram(const GramArgs& a, int io, int nt, int nr, hipStream_t s) {
  return io == IO_BF16 ? launch_gram_io<IO_BF16>(a, nt, nr, s)
                       : launch_gram_io<IO_F32>(a, nt, nr, s);
}

}  // namespace gdn
