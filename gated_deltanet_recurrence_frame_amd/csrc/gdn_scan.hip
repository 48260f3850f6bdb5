// Inter-frame propagation of the frame-wise GDN state.
//
// The recurrence S_t = S_{t-1} M_t + U_t with M_t = gamma_t I - A_t
// (summary page: 前置知识 "Gated DeltaNet" and 方法步骤详情 module 2) is
// evaluated as S_t = gamma_t S_{t-1} - S_{t-1} A_t + U_t.  M_t itself is
// never formed: at the default key scale A_t is ~1e-4 while gamma_t ~ 1,
// so gamma_t I - A_t would discard most of A_t's bits.
//
// Rows of S evolve independently (row i of S_t depends only on row i of
// S_{t-1}), so a workgroup owns 16 rows of one head's state and walks all T
// frames; the B*H*(D/16) workgroups of a launch are ordered so that the
// row blocks of one head share an XCD (and its L2 copy of A_t).  One wave
// per 16-column tile keeps its 16x16 tile of the state in fp32 registers.
// Per frame:
//   1. the tile is rounded to the intermediate type and staged in LDS, one
//      barrier, and every wave reads the 16 staged rows as the left MFMA
//      operand (the staged rows are also what is stored as S_{t-1});
//   2. P = Z A_t on MFMA (bf16 16x16x32, or fp32 16x16x4 for fp32 io).  A_t
//      is symmetric, so the right operand "column" k of tile j is row
//      16 j + i of A_t: each lane loads contiguous row pieces of A_t straight
//      from memory into registers;
//   3. Z <- gamma_t Z - P + U_t in fp32.
// The A_t pieces, the U_t tile and gamma_t of the next PD frames are in
// flight in a register ring while the current frame is processed, so the
// per-frame chain does not wait on memory latency.
//
// The reverse scan of the backward pass (adjoint of the recurrence,
// G_t = dO_t Q^_t^T + G_{t+1} M_{t+1}^T) runs the same code backwards in t:
// the input is added first, the sum is staged and stored, then multiplied
// by M_t.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT, bool REVERSE>
__global__ __launch_bounds__(64 * NT) void scan_kernel(ScanArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int KB = BF ? (D + 31) / 32 : D / 4;   // MFMA steps of one product
  constexpr int NAF = BF ? KB : D / 16;            // A pieces per lane per frame
  constexpr int PD = BF ? 8 : 3;                   // frames in flight
  constexpr int ZLD = BF ? D + 8 : D + 4;          // LDS row, a 16-byte multiple
  constexpr int GW = 512;                          // gamma window held in LDS
  constexpr int NTH = 64 * NT;
  typedef typename std::conditional<BF, bf16x8, f32x4>::type AF;
  typedef typename std::conditional<BF, u32x2, f32x4>::type UF;
  struct Buf {
    AF af[NAF];
    UF u;
  };
  __shared__ __attribute__((aligned(16))) E Zbuf[2][16 * ZLD];
  __shared__ float gam_lds[GW];

  const int total = a.B * a.H * NT;
  const int item = xcd_item(blockIdx.x, total);
  const int bh = item / NT, rb = item % NT;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), ct = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const long DD = (long)D * D;
  const int T = a.T;             // frames in the tensors
  const int NS = a.Tc;           // frames walked by this launch, from a.t0
  const E* Ab = static_cast<const E*>(a.A) + (long)bh * T * DD;
  const E* Ub = static_cast<const E*>(a.U) + (long)bh * T * DD;
  E* Eb = static_cast<E*>(a.emit) + (long)bh * T * DD;

  f32x4 z = zero4();
  if (a.z0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = a.z0[(long)bh * DD + (rb * 16 + 4 * g + r) * D + ct * 16 + li];
  }

  auto frame_of = [&](int s) { return REVERSE ? a.t0 + NS - 1 - s : a.t0 + s; };
  auto load = [&](Buf& B, int s) {
    const int t = frame_of(s < NS ? s : NS - 1);
    const E* At = Ab + t * DD + (ct * 16 + li) * D;
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k = kb * 32 + 8 * g;
        B.af[kb] = (k < D) ? load_bf16x8(At + k) : zero_bf16x8();
      }
      B.u = *reinterpret_cast<const u32x2*>(Ub + t * DD + ((rb * NT + ct) * 64 + lane) * 4);
    } else {
#pragma unroll
      for (int q = 0; q < NAF; ++q)
        B.af[q] = *reinterpret_cast<const f32x4*>(At + g * (D / 4) + 4 * q);
      B.u = *reinterpret_cast<const f32x4*>(Ub + t * DD + ((rb * NT + ct) * 64 + lane) * 4);
    }
  };
  auto unpack_u = [&](const Buf& B) -> f32x4 {
    if constexpr (BF) {
      f32x4 r;
      r[0] = bf16_bits_to_f32((uint16_t)(B.u[0] & 0xffff));
      r[1] = bf16_bits_to_f32((uint16_t)(B.u[0] >> 16));
      r[2] = bf16_bits_to_f32((uint16_t)(B.u[1] & 0xffff));
      r[3] = bf16_bits_to_f32((uint16_t)(B.u[1] >> 16));
      return r;
    } else {
      return B.u;
    }
  };
  auto stage = [&](int cur) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      E* dst = &Zbuf[cur][(4 * g + r) * ZLD + ct * 16 + li];
      if constexpr (BF)
        *dst = f32_to_bf16_bits(z[r]);
      else
        *dst = z[r];
    }
  };
  auto emit_rows = [&](int cur, int t) {   // the 16 staged rows -> S_t / G_t
    constexpr int PRW = D * ES / 16, NP = 16 * PRW;
    for (int p = tid; p < NP; p += NTH) {
      const int row = p / PRW, pc = p % PRW;
      *reinterpret_cast<u32x4*>(Eb + t * DD + (rb * 16 + row) * D + pc * (16 / ES)) =
          *reinterpret_cast<const u32x4*>(&Zbuf[cur][row * ZLD + pc * (16 / ES)]);
    }
  };
  auto load_gammas = [&](int s0) {
    for (int i = tid; i < GW; i += NTH) {
      const int s = s0 + i;
      gam_lds[i] = s < NS ? a.gamma[((long)b * T + frame_of(s)) * a.H + h] : 0.f;
    }
  };

  Buf ring[PD];
#pragma unroll
  for (int j = 0; j < PD; ++j) load(ring[j], j);

  for (int s0 = 0; s0 < NS; s0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int s = s0 + j;
      if (s < NS) {
        const int cur = s & 1;
        const int t = frame_of(s);
        if (s % GW == 0) {
          block_sync();
          load_gammas(s);
        }
        const f32x4 u = unpack_u(ring[j]);
        if constexpr (REVERSE) z += u;
        stage(cur);
        block_sync();
        const float gam = gam_lds[s % GW];
        if constexpr (REVERSE)
          emit_rows(cur, t);
        else if (s > 0)
          emit_rows(cur, t - 1);
        // P = Z[rows] A_t
        f32x4 p = zero4();
        const E* zrow = &Zbuf[cur][li * ZLD];
        if constexpr (BF) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int k = kb * 32 + 8 * g;
            const bf16x8 zf = (k < D) ? load_bf16x8(zrow + k) : zero_bf16x8();
            p = mfma_bf16(zf, ring[j].af[kb], p);
          }
        } else {
#pragma unroll
          for (int q = 0; q < NAF; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              p = mfma_f32(zrow[g * (D / 4) + 4 * q + e], ring[j].af[q][e], p);
        }
        if constexpr (REVERSE)
          z = gam * z - p;
        else
          z = gam * z - p + u;
        load(ring[j], s + PD);   // unconditional (clamped) keeps the compiler's wait counts exact
      }
    }
  }

  if constexpr (!REVERSE) {   // the walk's last state still has to be stored
    const int cur = NS & 1;
    stage(cur);
    block_sync();
    emit_rows(cur, a.t0 + NS - 1);
  }
  if (a.zT) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a.zT[(long)bh * DD + (rb * 16 + 4 * g + r) * D + ct * 16 + li] = z[r];
  }
}

template <int IO, int NT>
static hipError_t launch_scan_nt(const ScanArgs& a, bool reverse, hipStream_t s) {
  const dim3 grid(a.B * a.H * NT), block(64 * NT);
  if (reverse)
    hipLaunchKernelGGL((scan_kernel<IO, NT, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((scan_kernel<IO, NT, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_scan_io(const ScanArgs& a, int nt, bool reverse, hipStream_t s) {
  switch (nt) {
    case 1: return launch_scan_nt<IO, 1>(a, reverse, s);
    case 2: return launch_scan_nt<IO, 2>(a, reverse, s);
    case 3: return launch_scan_nt<IO, 3>(a, reverse, s);
    case 4: return launch_scan_nt<IO, 4>(a, reverse, s);
    case 5: return launch_scan_nt<IO, 5>(a, reverse, s);
    case 6: return launch_scan_nt<IO, 6>(a, reverse, s);
    case 7: return launch_scan_nt<IO, 7>(a, reverse, s);
    case 8: return launch_scan_nt<IO, 8>(a, reverse, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan(const ScanArgs& a, int io, int nt, bool reverse, hipStream_t s) {
  return io == IO_BF16 ? launch_scan_io<IO_BF16>(a, nt, reverse, s)
                       : launch_scan_io<IO_F32>(a, nt, reverse, s);
}

}  // namespace gdn
