// Output pass of the frame-wise GDN: O_t = S_t Q^_t (summary page,
// 方法步骤详情 module 2), i.e. o_{t,n} = S_t q_{t,n} for every token of the
// frame, with S_t the state after frame t's own update.
//
// One workgroup per (b, t, h) frame (XCD-aware order), one wave per 16-row
// feature tile of the output.  A wave keeps its 16 rows of S_t as MFMA
// operand fragments in registers for the whole frame (bf16: 4 x 8 values
// per lane at D = 112).  Query rows stream through LDS in chunks (natural
// [token][feature] layout, double-buffered, register prefetch of the next
// chunk); every wave reads the chunk's query rows as the other operand and
// writes its 16 features of each token (8-byte stores of 4 bf16).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT>
__global__ __launch_bounds__(64 * NT) void output_kernel(OutArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int CT = (IO == IO_BF16) ? 64 : 32;
  constexpr int PR = D * ES / 16;
  constexpr int PIECES = CT * PR;
  constexpr int NTH = 64 * NT;
  constexpr int PPT = (PIECES + NTH - 1) / NTH;
  constexpr int KB = (IO == IO_BF16) ? (D + 31) / 32 : D / 4;
  __shared__ __attribute__((aligned(16))) E tok[2][CT * D];

  const int total = a.B * a.T * a.H;
  const int item = xcd_item(blockIdx.x, total);
  const int h = item % a.H;
  const int t = (item / a.H) % a.T;
  const int b = item / (a.H * a.T);
  const int N = a.N;
  const long row0 = (long)b * a.T * N + (long)t * N;
  const int tid = threadIdx.x;
  const int lane = lane_id(), ft = wave_id();
  const int g = lane >> 4, li = lane & 15;

  // This wave's rows of S_t (intermediate type, row-major) as left MFMA
  // operands.
  const E* Sm = static_cast<const E*>(a.mat) + (((long)b * a.H + h) * a.T + t) * (long)(D * D) +
                (ft * 16 + li) * D;
  typedef typename std::conditional<IO == IO_BF16, bf16x8, float>::type Frag;
  Frag sf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if constexpr (IO == IO_BF16) {
      const int k = kb * 32 + 8 * g;
      sf[kb] = (k < D) ? load_bf16x8(Sm + k) : zero_bf16x8();
    } else {
      sf[kb] = Sm[kb * 4 + g];
    }
  }

  u32x4 pre[PPT];
  auto issue = [&](int c) {
    const int c0 = c * CT;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      if (p < PIECES) {
        const int row = p / PR, pc = p % PR;
        int tk = c0 + row;
        if (tk >= N) tk = N - 1;
        const E* src = static_cast<const E*>(a.tok) + ((row0 + tk) * a.H + h) * (long)D +
                       pc * (16 / ES);
        pre[j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };
  auto commit = [&](int stage) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      if (p < PIECES) *reinterpret_cast<u32x4*>(&tok[stage][p * (16 / ES)]) = pre[j];
    }
  };

  const int nchunks = (N + CT - 1) / CT;
  issue(0);
  commit(0);
  block_sync();
  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) issue(c + 1);
    const E* ts = tok[c & 1];
#pragma unroll
    for (int tt = 0; tt < CT / 16; ++tt) {
      f32x4 acc = zero4();
      const E* trow = ts + (tt * 16 + li) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (IO == IO_BF16) {
          const int k = kb * 32 + 8 * g;
          const bf16x8 q = (k < D) ? load_bf16x8(reinterpret_cast<const uint16_t*>(trow) + k)
                                   : zero_bf16x8();
          acc = mfma_bf16(sf[kb], q, acc);
        } else {
          acc = mfma_f32(sf[kb], reinterpret_cast<const float*>(trow)[kb * 4 + g], acc);
        }
      }
      const int tk = c * CT + tt * 16 + li;
      if (tk < N) {
        E* dst = static_cast<E*>(a.out) + ((row0 + tk) * a.H + h) * (long)D + ft * 16 + 4 * g;
        if constexpr (IO == IO_BF16) {
          u32x2 pk;
          pk[0] = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
          pk[1] = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
          *reinterpret_cast<u32x2*>(dst) = pk;
        } else {
          *reinterpret_cast<f32x4*>(dst) = acc;
        }
      }
    }
    if (c + 1 < nchunks) commit((c + 1) & 1);
    block_sync();
  }
}

template <int IO, int NT>
static hipError_t launch_output_nt(const OutArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((output_kernel<IO, NT>), dim3(a.B * a.T * a.H), dim3(64 * NT), 0, s, a);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_output_io(const OutArgs& a, int nt, hipStream_t s) {
  switch (nt) {
    case 1: return launch_output_nt<IO, 1>(a, s);
    case 2: return launch_output_nt<IO, 2>(a, s);
    case 3: return launch_output_nt<IO, 3>(a, s);
    case 4: return launch_output_nt<IO, 4>(a, s);
    case 5: return launch_output_nt<IO, 5>(a, s);
    case 6: return launch_output_nt<IO, 6>(a, s);
    case 7: return launch_output_nt<IO, 7>(a, s);
    case 8: return launch_output_nt<IO, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_output(const OutArgs& a, int io, int nt, hipStream_t s) {
  return io == IO_BF16 ? launch_output_io<IO_BF16>(a, nt, s) : launch_output_io<IO_F32>(a, nt, s);
}

}  // namespace gdn
