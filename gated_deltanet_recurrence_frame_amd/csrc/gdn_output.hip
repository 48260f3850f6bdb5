// Output pass of the frame-wise GDN: O_t = S_t Q^_t (summary page,
// 方法步骤详情 module 2), i.e. o_{t,n} = S_t q_{t,n} for every token of the
// frame, with S_t the state after frame t's own update.
//
// One workgroup per (b, t, h) frame (XCD-aware order), one wave per 16-row
// feature tile of the output.  A wave keeps its 16 rows of S_t as MFMA
// operand fragments in registers for the whole frame (bf16: 4 x 8 values
// per lane at D = 112).  Query rows stream through a 3-stage LDS ring in
// chunks (natural [token][feature] layout, copied straight from memory to
// LDS two chunks ahead); every wave reads the chunk's query rows as the
// other operand and stages its 16 features of each token in LDS; the next
// iteration stores the chunk's output rows as contiguous 16-byte pieces.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT, bool TRANS>
__global__ __launch_bounds__(64 * NT) void output_kernel(OutArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int CT = (IO == IO_BF16) ? 64 : 32;
  constexpr int MAT_BYTES = CT * D * ES;          // one chunk of query rows
  constexpr int WL = MAT_BYTES / 1024;            // 1 KB copies per chunk (= 2 NT)
  constexpr int OPS = WL / NT;                    // copies per wave per chunk
  constexpr int STAGES = 3;
  constexpr int KB = (IO == IO_BF16) ? (D + 31) / 32 : D / 4;
  constexpr int NTH = 64 * NT;
  static_assert(WL % NT == 0, "copies must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char ring[STAGES][MAT_BYTES];
  __shared__ __attribute__((aligned(16))) E obuf[2][CT * D];   // output chunk staging

  const int total = a.B * a.Tc * a.H * a.P;
  const int item = xcd_item(blockIdx.x, total);
  const int sp = item % a.P;                       // token split
  const int h = (item / a.P) % a.H;
  const int t = a.t0 + (item / (a.P * a.H)) % a.Tc;
  const int b = item / (a.P * a.H * a.Tc);
  const int N = a.N;
  const long row0 = (long)b * a.T * N + (long)t * N;
  const int lane = lane_id(), ft = wave_id();
  const int g = lane >> 4, li = lane & 15;

  // This wave's rows of the frame matrix (intermediate type, row-major in
  // memory) as left MFMA operands: rows of S_t, or with TRANS rows of
  // S_t^T (columns of S_t; the backward's dQ = S_t^T dO), which are staged
  // in LDS and read with the transposing LDS read.
  const E* Sm = static_cast<const E*>(a.mat) + (((long)b * a.H + h) * a.T + t) * (long)(D * D);
  typedef typename std::conditional<IO == IO_BF16, bf16x8, float>::type Frag;
  Frag sf[KB];
  if constexpr (!TRANS) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (IO == IO_BF16) {
        const int k = kb * 32 + 8 * g;
        sf[kb] = (k < D) ? load_bf16x8(Sm + (ft * 16 + li) * D + k) : zero_bf16x8();
      } else {
        sf[kb] = Sm[(ft * 16 + li) * D + kb * 4 + g];
      }
    }
  } else if constexpr (IO == IO_BF16) {
    // [KB*32][D] rows in the output staging area (free until the first
    // chunk), rows past D zero.
    uint16_t* ms = reinterpret_cast<uint16_t*>(&obuf[0][0]);
    constexpr int PRW = D / 8;
    for (int p = threadIdx.x; p < KB * 32 * PRW; p += NTH) {
      const int row = p / PRW, pc = p % PRW;
      *reinterpret_cast<u32x4*>(ms + row * D + pc * 8) =
          row < D ? *reinterpret_cast<const u32x4*>(Sm + row * D + pc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    block_sync();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb] = lds_col_frag_bf16(ms, D, kb * 32, ft * 16);
    block_sync();
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb] = Sm[(kb * 4 + g) * D + ft * 16 + li];
  }

  // Copy op i = ft + NT j of a chunk covers LDS bytes [1 KB i, +1 KB) of the
  // stage, lane l the 16 bytes at + 16 l (token row o / (D*ES)).
  const char* qsrc = static_cast<const char*>(a.tok);
  const int nchunks_all = (N + CT - 1) / CT;
  const int cps = (nchunks_all + a.P - 1) / a.P;  // chunks per split
  const int cbeg = sp * cps;
  const int nchunks = min(nchunks_all, cbeg + cps) - cbeg;
  if (nchunks <= 0) return;                        // before any barrier

  // local chunk c is frame chunk cbeg + c
  auto issue = [&](int c) {
    const int c0 = (cbeg + c) * CT;
#pragma unroll
    for (int j = 0; j < OPS; ++j) {
      const int i = ft + NT * j;
      const int o = i * 1024 + lane * 16;
      const int row = o / (D * ES), col = o % (D * ES);
      int tk = c0 + row;
      if (tk >= N) tk = N - 1;
      dma16(qsrc + (((row0 + tk) * a.H + h) * (long)D) * ES + col, &ring[c % STAGES][i * 1024]);
    }
  };

  // Output rows of a chunk are staged in LDS and stored one iteration later
  // as whole 16-byte pieces of token rows (each row of a head is D*ES
  // contiguous bytes), instead of 4 values per lane scattered over 16 rows.
  const int tid = threadIdx.x;
  auto store_chunk = [&](int c) {
    const E* src = obuf[c & 1];
    constexpr int PRW = D * ES / 16;
    for (int p = tid; p < CT * PRW; p += NTH) {
      const int row = p / PRW, pc = p % PRW;
      const int tk = (cbeg + c) * CT + row;
      if (tk < N)
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.out) + ((row0 + tk) * a.H + h) * (long)D +
                                  pc * (16 / ES)) =
            *reinterpret_cast<const u32x4*>(src + row * D + pc * (16 / ES));
    }
  };

#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c)
    if (c < nchunks) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    // Copies of chunk c+1 (if any) are younger than chunk c's; the output
    // stores in between only make the wait more conservative.
    if (c + 1 < nchunks)
      wait_vm_barrier<OPS>();
    else
      wait_vm_barrier<0>();
    if (c + STAGES - 1 < nchunks) issue(c + STAGES - 1);
    if (c > 0) store_chunk(c - 1);      // staged by every wave before the barrier
    const E* ts = reinterpret_cast<const E*>(ring[c % STAGES]);
    E* ob = obuf[c & 1];
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
      E* dst = ob + (tt * 16 + li) * D + ft * 16 + 4 * g;
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
  block_sync();
  store_chunk(nchunks - 1);
}

template <int IO, int NT, bool TRANS>
static hipError_t launch_output_nt(const OutArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((output_kernel<IO, NT, TRANS>), dim3(a.B * a.Tc * a.H * a.P), dim3(64 * NT),
                     0, s, a);
  return hipGetLastError();
}

template <int IO, bool TRANS>
static hipError_t launch_output_io(const OutArgs& a, int nt, hipStream_t s) {
  switch (nt) {
    case 1: return launch_output_nt<IO, 1, TRANS>(a, s);
    case 2: return launch_output_nt<IO, 2, TRANS>(a, s);
    case 3: return launch_output_nt<IO, 3, TRANS>(a, s);
    case 4: return launch_output_nt<IO, 4, TRANS>(a, s);
    case 5: return launch_output_nt<IO, 5, TRANS>(a, s);
    case 6: return launch_output_nt<IO, 6, TRANS>(a, s);
    case 7: return launch_output_nt<IO, 7, TRANS>(a, s);
    case 8: return launch_output_nt<IO, 8, TRANS>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_output(const OutArgs& a, int io, int nt, bool trans, hipStream_t s) {
  if (io == IO_BF16)
    return trans ? launch_output_io<IO_BF16, true>(a, nt, s) : launch_output_io<IO_BF16, false>(a, nt, s);
  return trans ? launch_output_io<IO_F32, true>(a, nt, s) : launch_output_io<IO_F32, false>(a, nt, s);
}

}  // namespace gdn
