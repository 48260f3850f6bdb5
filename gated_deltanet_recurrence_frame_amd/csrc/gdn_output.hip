// Output pass of the frame-wise GDN: O_t = S_t Q^_t (summary page,
// 方法步骤详情 module 2), i.e. o_{t,n} = S_t q_{t,n} for every token of the
// frame, with S_t the state after frame t's own update.  The backward's
// dQ^_t = S_t^T dO_t is the same pass on the transposed matrix.
//
// One workgroup per (b, t, h) frame (or per token range of it, for
// launches with few frames), XCD-aware order, one wave per 16-row feature
// tile of the output.  A wave keeps its 16 rows of S_t as MFMA operand
// fragments in registers for the whole frame.  Query rows stream in chunks
// of CT tokens: each thread loads two 16-byte pieces of a chunk (whole
// token rows per instruction) into a register ring PF chunks deep, commits
// them to LDS in the natural [token][feature] layout one chunk at a time,
// and every wave reads the chunk's query rows as the other MFMA operand.
// The outputs of a chunk are staged in LDS and stored one iteration later
// as contiguous 16-byte pieces of token rows.
//
// Query rows are read and output rows written non-temporally: they stream
// through once, and the caches keep the frame matrices (the scan's states,
// read just after they were written) instead.
// The ring is plain register loads that the compiler's wait counts track
// exactly (no direct-to-LDS copies, whose waits the compiler cannot relax
// while stores are pending), and the barriers are LDS-only, so the PF - 1
// chunks ahead stay in flight across them.  The loop over whole chunks is
// straight-line; the frame's last, partial chunk is finished after it.
// Normalised queries (NORM, forward only): o = S_t q / |q|, the
// accumulators scaled by 1 / |q| before rounding.  bf16: the query
// fragments of a 16-token tile are both operands of a second MFMA chain,
// whose result Q Q^T holds |q_i|^2 on its diagonal (lane (i / 4, i),
// register i % 4), read back by every lane of token i.  fp32: each lane
// sums the squares of its quarter of the features, added over the
// token's four lanes.  With inv_out the first wave also writes 1 / |q| of
// every token it scales (the forward keeps it in the saved buffer for the
// backward).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// bf16: registers kept to 128 so that two workgroups share a CU (4 waves per
// SIMD; the LDS stages allow it), which hides more of the per-chunk chain.
template <int IO, int NT, bool TRANS, int HPW, bool NORM>
__global__ __launch_bounds__(64 * NT, IO == IO_BF16 ? 4 : 1) void output_kernel(OutArgs a) {
  static_assert(!(NORM && TRANS), "normalised queries belong to the forward");
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int RW = HPW * D;                    // elements of a token's row segment
  constexpr int CT = (BF ? 64 : 32) / HPW;       // tokens per chunk
  constexpr int PR = RW * ES / 16;               // 16-byte pieces per row segment
  // LDS row stride: padded so that the 16 rows a fragment read (or an
  // output tile's write) touches start on different banks (row stride
  // = 4 mod 8 dwords: 116 dwords for bf16 head pairs of 112)
  constexpr int LDR = RW + (BF ? 8 : 4);
  constexpr int NTH = 64 * NT;
  constexpr int PPT = CT * PR / NTH;             // pieces per thread per chunk (2)
  constexpr int PF = 3;                          // chunks in flight
  static_assert(PPT * NTH == CT * PR, "pieces must split evenly over the threads");
  // contraction blocks: bf16 32-deep (the last one zero past D), fp32 4-deep
  constexpr int KF = BF ? (D + 31) / 32 : D / 4;
  constexpr bool KTAIL = BF && (D % 32) != 0;
  // (16 elements of padding: the zeroed tail of the last row's read stays in the array)
  __shared__ __attribute__((aligned(16))) E stage[2][CT * LDR + 16];
  __shared__ __attribute__((aligned(16))) E obuf[2][CT * LDR];

  const int HG = a.H / HPW;                        // head groups
  const int total = a.B * a.Tc * HG * a.P;
  const int item = xcd_item(blockIdx.x, total);
  const int sp = item % a.P;                       // token split
  const int h0 = ((item / a.P) % HG) * HPW;        // first head of the group
  const int t = a.t0 + (item / (a.P * HG)) % a.Tc;
  const int b = item / (a.P * HG * a.Tc);
  const int N = a.N;
  const long row0 = (long)b * a.T * N + (long)t * N;
  const int tid = threadIdx.x;
  const int lane = lane_id(), ft = wave_id();
  const int g = lane >> 4, li = lane & 15;

  const int nchunks_all = (N + CT - 1) / CT;
  const int cps = (nchunks_all + a.P - 1) / a.P;   // chunks per split
  const int cbeg = sp * cps;
  const int nchunks = min(nchunks_all, cbeg + cps) - cbeg;
  if (nchunks <= 0) return;                        // whole workgroup, before any barrier

  // This wave's rows of each head's frame matrix as left MFMA operands:
  // rows of S_t, or with TRANS rows of S_t^T (columns of S_t), read from
  // S_t staged in LDS with the transposing LDS read.
  typedef typename std::conditional<BF, bf16x8, float>::type Frag;
  Frag sf[HPW][KF];
#pragma unroll
  for (int hp = 0; hp < HPW; ++hp) {
    const E* Sm = static_cast<const E*>(a.mat) + (((long)b * a.H + h0 + hp) * a.T + t) * (long)(D * D);
    if constexpr (!TRANS) {
      if constexpr (BF) {
        const E* row = Sm + (ft * 16 + li) * D;
#pragma unroll
        for (int kb = 0; kb < KF; ++kb) {
          const int k = kb * 32 + 8 * g;
          sf[hp][kb] = (k < D) ? load_bf16x8(row + k) : zero_bf16x8();
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KF; ++kb) sf[hp][kb] = Sm[(ft * 16 + li) * D + kb * 4 + g];
      }
    } else if constexpr (BF) {
      // S_t as [KR][D] rows in the output staging (free until the first
      // chunk), rows past D zero
      constexpr int KR = KF * 32;
      static_assert(KR * D <= 2 * CT * LDR, "staged matrix must fit the output buffers");
      uint16_t* ms = reinterpret_cast<uint16_t*>(&obuf[0][0]);
      constexpr int PRW = D / 8;
      for (int p = tid; p < KR * PRW; p += NTH) {
        const int row = p / PRW, pc = p % PRW;
        *reinterpret_cast<u32x4*>(ms + row * D + pc * 8) =
            row < D ? *reinterpret_cast<const u32x4*>(Sm + row * D + pc * 8) : u32x4{0u, 0u, 0u, 0u};
      }
      block_sync();
#pragma unroll
      for (int kb = 0; kb < KF; ++kb) sf[hp][kb] = lds_col_frag_bf16(ms, D, kb * 32, ft * 16);
      block_sync();
    } else {
#pragma unroll
      for (int kb = 0; kb < KF; ++kb) sf[hp][kb] = Sm[(kb * 4 + g) * D + ft * 16 + li];
    }
  }

  const E* tok = static_cast<const E*>(a.tok);
  E* out = static_cast<E*>(a.out);
  struct Ring {
    u32x4 v[PPT];
  };
  // Local chunk c is frame chunk cbeg + c; rows past the frame re-read its
  // last row.  A row segment is the HPW adjacent heads' D features of one
  // token (contiguous in memory).
  auto issue = [&](Ring& R, int c) {
    const int c0 = (cbeg + (c < nchunks ? c : nchunks - 1)) * CT;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      const int row = p / PR, pc = p % PR;
      int tk = c0 + row;
      if (tk >= N) tk = N - 1;
      R.v[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(tok + ((row0 + tk) * a.H + h0) * (long)D + pc * (16 / ES)));
    }
  };
  auto commit = [&](const Ring& R, int c) {
    E* st = stage[c & 1];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      *reinterpret_cast<u32x4*>(st + (p / PR) * LDR + (p % PR) * (16 / ES)) = R.v[j];
    }
  };
  auto compute = [&](int c) {
    const E* ts = stage[c & 1];
    E* ob = obuf[c & 1];
#pragma unroll
    for (int hp = 0; hp < HPW; ++hp)
#pragma unroll
      for (int tt = 0; tt < CT / 16; ++tt) {
        f32x4 acc = zero4();
        const E* trow = ts + (tt * 16 + li) * LDR + hp * D;
        float ss = 0.f;   // NORM: |q|^2 of this lane's token (fp32: its share)
        if constexpr (BF) {
          f32x4 gram = zero4();   // NORM: Q Q^T of the tile's 16 tokens
#pragma unroll
          for (int kb = 0; kb < KF; ++kb) {
            // past D the read runs into the next head or row (or the next
            // LDS buffer): zero it, the matching operand is zero too
            bf16x8 q = load_bf16x8(reinterpret_cast<const uint16_t*>(trow) + kb * 32 + 8 * g);
            if (KTAIL && kb == KF - 1 && kb * 32 + 8 * g >= D) q = zero_bf16x8();
            acc = mfma_bf16(sf[hp][kb], q, acc);
            if constexpr (NORM) gram = mfma_bf16(q, q, gram);
          }
          if constexpr (NORM) {
            const int r = li & 3;
            const float dg = r == 0 ? gram[0] : r == 1 ? gram[1] : r == 2 ? gram[2] : gram[3];
            ss = __shfl(dg, ((li >> 2) << 4) | li);   // lane (i / 4, i)
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < KF; ++kb) {
            const float x = trow[kb * 4 + g];
            acc = mfma_f32(sf[hp][kb], x, acc);
            if constexpr (NORM) ss = fmaf(x, x, ss);
          }
        }
        if constexpr (NORM) {   // token tt * 16 + i sits in lanes i, i + 16, i + 32, i + 48
          if constexpr (!BF) {
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
          }
          const float iv = inv_norm(ss);
          acc *= iv;
          // 1 / |q| per row for the backward (every wave has it; the first writes)
          const int tq = (cbeg + c) * CT + tt * 16 + li;
          if (a.inv_out && ft == 0 && g == 0 && tq < N) a.inv_out[(row0 + tq) * a.H + h0 + hp] = iv;
        }
        E* dst = ob + (tt * 16 + li) * LDR + hp * D + ft * 16 + 4 * g;
        if constexpr (BF) {
          u32x2 pk;
          pk[0] = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
          pk[1] = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
          *reinterpret_cast<u32x2*>(dst) = pk;
        } else {
          *reinterpret_cast<f32x4*>(dst) = acc;
        }
      }
  };
  auto store_full = [&](int c) {   // every token of chunk c exists
    const E* src = obuf[c & 1];
    const long r0 = row0 + (long)(cbeg + c) * CT;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      const int row = p / PR, pc = p % PR;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src + row * LDR + pc * (16 / ES)),
                                  reinterpret_cast<u32x4*>(out + ((r0 + row) * a.H + h0) * (long)D +
                                                           pc * (16 / ES)));
    }
  };
  auto store_tail = [&](int c) {
    const E* src = obuf[c & 1];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      const int row = p / PR, pc = p % PR;
      const int tk = (cbeg + c) * CT + row;
      if (tk < N)
        *reinterpret_cast<u32x4*>(out + ((row0 + tk) * a.H + h0) * (long)D + pc * (16 / ES)) =
            *reinterpret_cast<const u32x4*>(src + row * LDR + pc * (16 / ES));
    }
  };

  // the frame's chunks before its last are whole; the last may be partial
  const int nfull = ((cbeg + nchunks) * CT <= N) ? nchunks : nchunks - 1;

  Ring ring[PF];
#pragma unroll
  for (int r = 0; r < PF; ++r) issue(ring[r], r);
  // chunk 0: nothing to store yet
  commit(ring[0], 0);
  lds_barrier();
  issue(ring[0], PF);
  compute(0);
  // chunks 1 .. : straight-line trips of PF chunks while all are whole
  int c0 = 1;
  for (; c0 + PF <= nfull; c0 += PF) {
#pragma unroll
    for (int r = 0; r < PF; ++r) {
      const int c = c0 + r;
      Ring& R = ring[(1 + r) % PF];
      commit(R, c);
      lds_barrier();
      issue(R, c + PF);        // clamped past the end
      store_full(c - 1);
      compute(c);
    }
  }
#pragma unroll
  for (int r = 0; r < PF; ++r) {
    const int c = c0 + r;
    if (c < nchunks) {
      commit(ring[(1 + r) % PF], c);
      lds_barrier();
      store_full(c - 1);       // not the last chunk
      compute(c);
    }
  }
  lds_barrier();
  if (nfull == nchunks)
    store_full(nchunks - 1);
  else
    store_tail(nchunks - 1);
}

template <int IO, int NT, bool TRANS, bool NORM>
static hipError_t launch_output_norm(const OutArgs& a, hipStream_t s) {
  // adjacent head pairs when H is even: 2 D-wide row segments per token are
  // contiguous and 64-byte aligned, where one head's rows are not
  if (a.H % 2 == 0)
    hipLaunchKernelGGL((output_kernel<IO, NT, TRANS, 2, NORM>), dim3(a.B * a.Tc * (a.H / 2) * a.P),
                       dim3(64 * NT), 0, s, a);
  else
    hipLaunchKernelGGL((output_kernel<IO, NT, TRANS, 1, NORM>), dim3(a.B * a.Tc * a.H * a.P),
                       dim3(64 * NT), 0, s, a);
  return hipGetLastError();
}

template <int IO, int NT, bool TRANS>
static hipError_t launch_output_nt(const OutArgs& a, hipStream_t s) {
  if constexpr (TRANS) {
    if (a.norm) return hipErrorInvalidValue;
    return launch_output_norm<IO, NT, true, false>(a, s);
  } else {
    return a.norm ? launch_output_norm<IO, NT, false, true>(a, s)
                  : launch_output_norm<IO, NT, false, false>(a, s);
  }
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
