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
//      from memory into registers.  bf16 A_t is stored in that operand order
//      (the fragment layout), so a wave's load of one 32-column block is one
//      contiguous 1 KB piece: a third fewer cycles per frame than loading
//      row pieces from a row-major A_t, whose 64-byte runs spread every
//      load over 16 rows;
//   3. Z <- gamma_t Z - P + U_t in fp32.
// The A_t pieces, the U_t tile and gamma_t of the next PD frames are in
// flight in a register ring while the current frame is processed, so the
// per-frame chain does not wait on memory latency.
//
// The reverse scan of the backward pass (adjoint of the recurrence,
// G_t = dO_t Q^_t^T + G_{t+1} M_{t+1}^T) runs the same code backwards in t:
// the input is added first, the sum is staged and stored, then multiplied
// by M_t.
//
// Chunked mode (the transition / input composites of the context-parallel
// scheme, summary page 技术新颖性 point 1, with chunks of frames in place
// of devices): the composite walk keeps 32 staged rows, 16 of the input
// composite H (from zero, with the inputs) and 16 of the transition
// composite C (from the identity, without them), which share every A_t
// fragment.  C is kept in fp32 registers and stored in fp32; it is never
// rounded to the intermediate type except as an MFMA operand, like S.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT, int MODE>
__global__ __launch_bounds__(64 * NT) void scan_kernel(ScanArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr bool REVERSE = (MODE & 1) != 0;
  constexpr bool COMP = (MODE & 2) != 0;   // composite: H and C walked together
  constexpr int ZR = COMP ? 32 : 16;       // staged rows (H rows, then C rows)
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int KB = BF ? (D + 31) / 32 : D / 4;   // MFMA steps of one product
  constexpr int NAF = BF ? KB : D / 16;            // A pieces per lane per frame
  constexpr int PD = BF ? 8 : 3;                   // frames in flight
  constexpr int ZLD = BF ? D + 8 : D + 4;          // LDS row, a 16-byte multiple
  constexpr int NTH = 64 * NT;
  typedef typename std::conditional<BF, bf16x8, f32x4>::type AF;
  typedef typename std::conditional<BF, u32x2, f32x4>::type UF;
  struct Buf {
    AF af[NAF];
    UF u;
    float gm;
  };
  __shared__ __attribute__((aligned(16))) E Zbuf[2][ZR * ZLD];

  const int NW = a.Tc;                                // frames of the whole walk
  const int CH = a.chunk > 0 ? a.chunk : NW;
  const int nck = (NW + CH - 1) / CH;
  const int total = a.B * a.H * nck * NT;
  const int item = xcd_item(blockIdx.x, total);
  const int rb = item % NT;
  const int w = (item / NT) % nck;                    // chunk, in walk order
  const int bh = item / NT / nck;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), ct = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const long DD = (long)D * D;
  const int T = a.T;                                  // frames in the tensors
  const int sb = w * CH;                              // first walk step of the chunk
  const int NS = NW - sb < CH ? NW - sb : CH;         // steps walked here
  const E* Ab = static_cast<const E*>(a.A) + (long)bh * T * DD;
  const E* Ub = static_cast<const E*>(a.U) + (long)bh * T * DD;
  E* Eb = static_cast<E*>(a.emit) + (long)bh * T * DD;

  f32x4 z = zero4();
  f32x4 zc = zero4();   // COMP: the transition composite, from the identity
  if constexpr (COMP) {
#pragma unroll
    for (int r = 0; r < 4; ++r) zc[r] = (rb * 16 + 4 * g + r == ct * 16 + li) ? 1.f : 0.f;
  } else {
    const float* zs = a.chunk > 0 ? a.zmid + ((long)bh * nck + w) * DD
                                  : (a.z0 ? a.z0 + (long)bh * DD : nullptr);
    if (zs) {
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = zs[(rb * 16 + 4 * g + r) * D + ct * 16 + li];
    }
  }

  // gamma_t rides in the ring with A_t and U_t.  Without gates (the fold
  // of the composites, fp32) the load reads the first element of A instead
  // (finite) and the state is scaled by gz = 0 before it meets it.  Nothing
  // is applied to a loaded value until its frame is processed: an operation
  // on it alone (a select) is free to be scheduled right after the load and
  // would wait for it there.
  const bool gated = a.gamma != nullptr;
  const float* gbase = gated ? a.gamma + (long)b * T * a.H + h : static_cast<const float*>(a.A);
  const int gstride = gated ? a.H : 0;
  const float gz = gated ? 1.f : 0.f;

  auto frame_of = [&](int s) { return REVERSE ? a.t0 + NW - 1 - (sb + s) : a.t0 + sb + s; };
  auto load = [&](Buf& B, int s) {
    const int t = frame_of(s < NS ? s : NS - 1);
    B.gm = gbase[(long)t * gstride];
    if constexpr (BF) {
      // this wave's 16-row block of A_t in the fragment layout: block kb is
      // 64 lanes x 8 elements (fewer lanes' worth for a last block of 16
      // columns).  Unconditional loads: a branch around a load would cost
      // the compiler its count of loads in flight and drain the ring every
      // frame.  Lanes whose columns run past D re-read another lane's 8
      // elements of the block (finite); the staged-row operand is zero
      // there, so they add exact zeros.
      const E* Af = Ab + t * DD + ct * 16 * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int kw = min(4, (D - kb * 32) / 8);   // 8-column groups inside D
        const int gc = g < kw ? g : kw - 1;
        B.af[kb] = load_bf16x8(Af + kb * 512 + (16 * gc + li) * 8);
      }
      B.u = *reinterpret_cast<const u32x2*>(Ub + t * DD + ((rb * NT + ct) * 64 + lane) * 4);
    } else {
      const E* At = Ab + t * DD + (ct * 16 + li) * D;
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
  auto stage_tile = [&](int cur, int row0, const f32x4& v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      E* dst = &Zbuf[cur][(row0 + 4 * g + r) * ZLD + ct * 16 + li];
      if constexpr (BF)
        *dst = f32_to_bf16_bits(v[r]);
      else
        *dst = v[r];
    }
  };
  // the 16 staged rows -> S_t / G_t: 16 D elements, exactly 4 per thread,
  // one unconditional store each (no branch around the store)
  auto emit_rows = [&](int cur, int t) {
    constexpr int PRW = D / 4;                     // 4-element pieces per row
    static_assert(16 * PRW == NTH, "one piece per thread");
    const int row = tid / PRW, pc = tid % PRW;
    typedef typename std::conditional<BF, u32x2, u32x4>::type P4;
    *reinterpret_cast<P4*>(Eb + t * DD + (rb * 16 + row) * D + pc * 4) =
        *reinterpret_cast<const P4*>(&Zbuf[cur][row * ZLD + pc * 4]);
  };
  auto product = [&](const E* zrow, const Buf& B) {   // staged rows x A_t
    f32x4 p = zero4();
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k = kb * 32 + 8 * g;
        const bf16x8 zf = (k < D) ? load_bf16x8(zrow + k) : zero_bf16x8();
        p = mfma_bf16(zf, B.af[kb], p);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NAF; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p = mfma_f32(zrow[g * (D / 4) + 4 * q + e], B.af[q][e], p);
    }
    return p;
  };

  // One frame of the walk (step s, ring slot j = s % PD): add the input
  // first in the reverse walk, stage the rows, barrier, store the staged rows
  // (S_{t-1} / G_t), multiply by A_t, update, reload the slot PD frames
  // ahead.
  auto step = [&](Buf& R, int s, bool first) {
    const int cur = s & 1;
    const int t = frame_of(s);
    const float gam = R.gm;   // multiplies gz * state, never alone
    const f32x4 u = unpack_u(R);
    if constexpr (REVERSE) z += u;
    stage_tile(cur, 0, z);
    if constexpr (COMP) stage_tile(cur, 16, zc);
    block_sync();
    if constexpr (!COMP) {
      if constexpr (REVERSE)
        emit_rows(cur, t);
      else
        // the staged rows are the state before frame t, stored at t - 1;
        // at the walk's first frame (nothing to store unless asked) they go
        // to frame t's own slot instead, which the same threads overwrite
        // with S_t one step later - a select, not a branch around the store
        emit_rows(cur, (!first || a.emit_entry) ? t - 1 : t);
    }
    // P = Z[rows] A_t
    const f32x4 p = product(&Zbuf[cur][li * ZLD], R);
    if constexpr (COMP) {
      const f32x4 pc = product(&Zbuf[cur][(16 + li) * ZLD], R);
      zc = gam * (gz * zc) - pc;
    }
    if constexpr (REVERSE)
      z = gam * (gz * z) - p;
    else
      z = gam * (gz * z) - p + u;
    load(R, s + PD);   // unconditional (clamped)
  };

  // The first frame runs on its own; then whole trips of PD frames run
  // without any branch around a memory operation (the compiler then keeps
  // exact counts of the loads in flight and waits only for the slot it
  // needs); the last, partial trip follows.
  Buf ring[PD];
#pragma unroll
  for (int j = 0; j < PD; ++j) load(ring[j], j);
  step(ring[0], 0, true);
  int s0 = 1;
  for (; s0 + PD <= NS; s0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) step(ring[(1 + j) % PD], s0 + j, false);
  }
#pragma unroll
  for (int j = 0; j < PD; ++j)
    if (s0 + j < NS) step(ring[(1 + j) % PD], s0 + j, false);

  if constexpr (COMP) {
    float* Hd = a.compH + ((long)bh * nck + w) * DD + ((rb * NT + ct) * 64 + lane) * 4;
    *reinterpret_cast<f32x4*>(Hd) = z;
    float* Cd = a.compC + ((long)bh * nck + w) * DD + (ct * 16 + li) * D + rb * 16 + 4 * g;
    *reinterpret_cast<f32x4*>(Cd) = -zc;
  } else {
    if constexpr (!REVERSE) {   // the walk's last state still has to be stored
      const int cur = NS & 1;
      stage_tile(cur, 0, z);
      block_sync();
      emit_rows(cur, frame_of(NS - 1));
    }
    if (a.zT && w == nck - 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) a.zT[(long)bh * DD + (rb * 16 + 4 * g + r) * D + ct * 16 + li] = z[r];
    }
  }
}

template <int IO, int NT>
static hipError_t launch_scan_nt(const ScanArgs& a, int mode, hipStream_t s) {
  const int ch = a.chunk > 0 ? a.chunk : a.Tc;
  const int nck = (a.Tc + ch - 1) / ch;
  const dim3 grid(a.B * a.H * nck * NT), block(64 * NT);
  switch (mode) {
    case SCAN_FWD: hipLaunchKernelGGL((scan_kernel<IO, NT, SCAN_FWD>), grid, block, 0, s, a); break;
    case SCAN_REV: hipLaunchKernelGGL((scan_kernel<IO, NT, SCAN_REV>), grid, block, 0, s, a); break;
    case SCAN_COMP_FWD:
      hipLaunchKernelGGL((scan_kernel<IO, NT, SCAN_COMP_FWD>), grid, block, 0, s, a);
      break;
    case SCAN_COMP_REV:
      hipLaunchKernelGGL((scan_kernel<IO, NT, SCAN_COMP_REV>), grid, block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_scan_io(const ScanArgs& a, int nt, int mode, hipStream_t s) {
  switch (nt) {
    case 1: return launch_scan_nt<IO, 1>(a, mode, s);
    case 2: return launch_scan_nt<IO, 2>(a, mode, s);
    case 3: return launch_scan_nt<IO, 3>(a, mode, s);
    case 4: return launch_scan_nt<IO, 4>(a, mode, s);
    case 5: return launch_scan_nt<IO, 5>(a, mode, s);
    case 6: return launch_scan_nt<IO, 6>(a, mode, s);
    case 7: return launch_scan_nt<IO, 7>(a, mode, s);
    case 8: return launch_scan_nt<IO, 8>(a, mode, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan(const ScanArgs& a, int io, int nt, int mode, hipStream_t s) {
  if (a.Tc < 1) return hipErrorInvalidValue;
  return io == IO_BF16 ? launch_scan_io<IO_BF16>(a, nt, mode, s)
                       : launch_scan_io<IO_F32>(a, nt, mode, s);
}

}  // namespace gdn
