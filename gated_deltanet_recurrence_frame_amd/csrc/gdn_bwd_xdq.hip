// The backward's pass over dO (chain rule of the summary page's module-2
// recurrence, O_t = S_t Q^_t): for each (b, t) frame and group of HPW
// adjacent heads, in one stream over the frame's dO and Q rows,
//   X_t   = dO_t Q^_t^T     the frame's own contribution to dLoss/dS_t,
//                           the input of the reverse scan;
//   dQ^_t = S_t^T dO_t      the gradient of the queries.
// Both products read every dO row; as one pass they read dO once instead of
// twice (the Gram-mode X pass and the transposed output pass, which remain
// for fp32 and for launches of few frames).
//
// One workgroup per item, one wave per (head, 16-feature tile).  Each wave
// keeps its 16 rows of S_t^T (columns of S_t, staged in LDS once and read
// with the transposing LDS read) as MFMA operands in registers.  dO and Q
// rows stream in chunks of 32 tokens through a register ring into a
// double-buffered LDS stage (LDS-only barriers, so the ring stays in flight
// across them):
//   X:  the wave's 16 dO features over the chunk's 32 tokens (transposing
//       read) against every 16-feature tile of Q, one 32-deep MFMA each,
//       accumulated over the frame in fp32;
//   dQ: S_t^T rows against the chunk's dO rows (plain 16-byte reads), staged
//       in LDS and stored one chunk later as contiguous 16-byte pieces of
//       token rows.
// dO rows past the frame's end are zeroed when staged, so they add nothing
// to X (their dQ rows are not stored).
//
// With normalised queries (CHAIN) the pass reads the raw query rows and
// 1 / |q| per row (summary page, 方法步骤详情 module 2, the hats read as
// per-token normalisation): each thread stages its piece as q^ = q / |q|
// (bf16), and dQ^ goes through the normalisation's chain rule before it is
// stored, dq = (dq^ - q^ (q^ . dq^)) / |q|.  Each wave adds q^ . dq^ over its
// 16 features of a token; the stores sum the tiles' partials in a fixed
// order (deterministic) and apply the rule to whole 16-byte pieces.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// LDS row stride (bf16 elements) for the transposing reads: 4 consecutive
// rows per lane group on different banks (stride 8 or 24 dwords mod 32).
constexpr int xdq_pad(int rw) {
  for (int p = 0; p < 64; p += 8) {
    const int sd = (rw + p) / 2;
    if (sd % 32 == 8 || sd % 32 == 24) return rw + p;
  }
  return rw;
}

template <int NT, int HPW, bool CHAIN>
__global__ __launch_bounds__(64 * NT * HPW, 1) void xdq_kernel(XdqArgs a) {
  constexpr int D = 16 * NT;
  constexpr int RW = HPW * D;               // elements of a token's row segment
  constexpr int CT = 32;                    // tokens per chunk: one 32-deep X step
  constexpr int PR = RW / 8;                // 16-byte pieces per row segment
  constexpr int NTH = 64 * NT * HPW;
  static_assert(CT * PR == NTH, "one piece of each matrix per thread per chunk");
  constexpr int PF = 2;                     // chunks in flight
  constexpr int KB = (D + 31) / 32;
  constexpr bool KTAIL = (D % 32) != 0;
  constexpr int LDR = xdq_pad(RW);          // stage rows
  constexpr int LDO = RW + 8;               // output rows (4 mod 8 dwords)
  constexpr int KR = KB * 32;               // staged rows of S_t (zero past D)
  constexpr int STAGE = 2 * CT * LDR + 16;  // dO rows, Q rows (+ the zeroed tail's reach)
  static_assert(HPW * KR * D <= 2 * STAGE, "S_t of the group must fit the stage");
  __shared__ __attribute__((aligned(16))) uint16_t stage[2][STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t obuf[2][CT * LDO];
  // CHAIN: q^ . dq^ per (head, tile, token); 1 / |q| of each thread's piece
  // (per token, the tiles' partials side by side: the store reads them as
  // two 16-byte pieces)
  __shared__ __attribute__((aligned(16))) float cred[CHAIN ? 2 : 1][HPW][CT][8];
  static_assert(NT <= 8, "the partials' row holds eight tiles");
  __shared__ float istage[CHAIN ? 2 : 1][CHAIN ? NTH : 1];

  const int HG = a.H / HPW;
  const int total = a.B * a.T * HG;
  const int item = xcd_item(blockIdx.x, total);
  const int h0 = (item % HG) * HPW;
  const int t = (item / HG) % a.T;
  const int b = item / (HG * a.T);
  const int N = a.N;
  const long row0 = (long)b * a.T * N + (long)t * N;
  const long DD = (long)D * D;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int hp = wave / NT, ft = wave % NT;
  const int g = lane >> 4, li = lane & 15;

  // S_t^T rows of this wave's tile: S_t of the group's heads staged as
  // [KR][D] rows, read by columns.
  bf16x8 sf[KB];
  {
    uint16_t* ms = &stage[0][0];
    constexpr int PRW = D / 8;
    for (int p = tid; p < HPW * KR * PRW; p += NTH) {
      const int m = p / (KR * PRW), r = p % (KR * PRW);
      const int row = r / PRW, pc = r % PRW;
      const uint16_t* Sm = static_cast<const uint16_t*>(a.S) +
                           (((long)b * a.H + h0 + m) * a.T + t) * DD;
      *reinterpret_cast<u32x4*>(ms + (m * KR + row) * D + pc * 8) =
          row < D ? *reinterpret_cast<const u32x4*>(Sm + row * D + pc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    block_sync();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb] = lds_col_frag_bf16(ms + hp * KR * D, D, kb * 32, ft * 16);
    block_sync();
  }

  // a uniform 64-bit base of the frame's rows plus 32-bit per-lane offsets
  // (the host keeps a frame's rows under 2 GiB and N, H D 2 under 2^24)
  const long fbase = (row0 * a.H + h0) * (long)(D * 2);
  const char* dob = static_cast<const char*>(a.d_o) + fbase;
  const char* qb = static_cast<const char*>(a.q) + fbase;
  char* dqb = static_cast<char*>(a.dq) + fbase;
  const unsigned rowb = (unsigned)(a.H * D * 2);
  const int nchunks = (N + CT - 1) / CT;
  const int prow = tid / PR, ppc = tid % PR;    // this thread's piece of a chunk

  struct Ring {
    u32x4 o, q;
    float iv;   // CHAIN: 1 / |q| of this thread's piece (token, head)
  };
  auto issue = [&](Ring& R, int c) {
    int tk = (c < nchunks ? c : nchunks - 1) * CT + prow;
    if (tk >= N) tk = N - 1;
    const unsigned off = __umul24((unsigned)tk, rowb) + (unsigned)(ppc * 16);
    R.o = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dob + off));
    R.q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qb + off));
    if constexpr (CHAIN) R.iv = a.inv[(row0 + tk) * a.H + h0 + ppc / (D / 8)];
  };
  auto commit = [&](const Ring& R, int c) {
    uint16_t* st = stage[c & 1];
    const bool live = c * CT + prow < N;        // rows past the frame: dO zero
    *reinterpret_cast<u32x4*>(st + prow * LDR + ppc * 8) = live ? R.o : u32x4{0u, 0u, 0u, 0u};
    if constexpr (CHAIN) {
      *reinterpret_cast<u32x4*>(st + (CT + prow) * LDR + ppc * 8) = piece_scale<IO_BF16>(R.q, R.iv);
      istage[c & 1][tid] = R.iv;   // read back by this thread when it stores the chunk
    } else {
      *reinterpret_cast<u32x4*>(st + (CT + prow) * LDR + ppc * 8) = R.q;
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) acc[ct] = zero4();
  auto compute = [&](int c) {
    const uint16_t* ds = stage[c & 1] + hp * D;
    const uint16_t* qs = stage[c & 1] + CT * LDR + hp * D;
    // X += dO^T Q over the chunk's 32 tokens
    const bf16x8 af = lds_col_frag_bf16(ds, LDR, 0, ft * 16);
    // (a few fragments live at a time: 14 waves per CU leave a wave 128
    // registers, of which the X accumulators take 4 NT)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      acc[ct] = mfma_bf16(af, lds_col_frag_bf16(qs, LDR, 0, ct * 16), acc[ct]);
      if (ct % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // dQ rows of the chunk's two 16-token tiles
    uint16_t* ob = obuf[c & 1];
#pragma unroll 1
    for (int tt = 0; tt < CT / 16; ++tt) {
      const int trow = tt * 16 + li;
      f32x4 d = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // past D the read runs into the next head or the padding: zero it
        bf16x8 o = load_bf16x8(ds + trow * LDR + kb * 32 + 8 * g);
        if (KTAIL && kb == KB - 1 && kb * 32 + 8 * g >= D) o = zero_bf16x8();
        d = mfma_bf16(sf[kb], o, d);
      }
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(d[0]) | ((uint32_t)f32_to_bf16_bits(d[1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(d[2]) | ((uint32_t)f32_to_bf16_bits(d[3]) << 16);
      *reinterpret_cast<u32x2*>(ob + trow * LDO + hp * D + ft * 16 + 4 * g) = pk;
      if constexpr (CHAIN) {
        // q^ . dq^ over this wave's 16 features of the token (lanes li,
        // li + 16, li + 32, li + 48 hold 4 each)
        const u32x2 qp = *reinterpret_cast<const u32x2*>(qs + trow * LDR + ft * 16 + 4 * g);
        float part = bf16_bits_to_f32((uint16_t)(qp[0] & 0xffff)) * d[0];
        part += bf16_bits_to_f32((uint16_t)(qp[0] >> 16)) * d[1];
        part += bf16_bits_to_f32((uint16_t)(qp[1] & 0xffff)) * d[2];
        part += bf16_bits_to_f32((uint16_t)(qp[1] >> 16)) * d[3];
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (g == 0) cred[c & 1][hp][trow][ft] = part;
      }
    }
  };
  auto store = [&](int c, bool full) {
    const int tk = c * CT + prow;
    u32x4 v = *reinterpret_cast<const u32x4*>(&obuf[c & 1][prow * LDO + ppc * 8]);
    if constexpr (CHAIN) {
      // dq = (dq^ - q^ (q^ . dq^)) / |q| on this piece of head hm's row
      const int hm = ppc / (D / 8);
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(&cred[c & 1][hm][prow][0]);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(&cred[c & 1][hm][prow][4]);
      const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      float dot = 0.f;
#pragma unroll
      for (int f = 0; f < NT; ++f) dot += cv[f];
      const float iv = istage[c & 1][tid];
      const u32x4 qv = *reinterpret_cast<const u32x4*>(&stage[c & 1][(CT + prow) * LDR + ppc * 8]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g0 = __uint_as_float(v[e] << 16), g1 = __uint_as_float(v[e] & 0xffff0000u);
        const float q0 = __uint_as_float(qv[e] << 16), q1 = __uint_as_float(qv[e] & 0xffff0000u);
        v[e] = (uint32_t)f32_to_bf16_bits((g0 - q0 * dot) * iv) |
               ((uint32_t)f32_to_bf16_bits((g1 - q1 * dot) * iv) << 16);
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(dqb + __umul24((unsigned)tk, rowb) + (unsigned)(ppc * 16));
    if (full || tk < N) __builtin_nontemporal_store(v, dst);
  };

  // chunks before the frame's last are whole; the last may be partial
  const int nfull = (nchunks * CT <= N) ? nchunks : nchunks - 1;
  Ring ring[PF];
#pragma unroll
  for (int r = 0; r < PF; ++r) issue(ring[r], r);
  commit(ring[0], 0);
  lds_barrier();
  issue(ring[0], PF);
  compute(0);
  int c0 = 1;
  for (; c0 + PF <= nfull; c0 += PF) {
#pragma unroll
    for (int r = 0; r < PF; ++r) {
      const int c = c0 + r;
      Ring& R = ring[(1 + r) % PF];
      commit(R, c);
      lds_barrier();
      issue(R, c + PF);        // clamped past the end
      store(c - 1, true);
      compute(c);
    }
  }
#pragma unroll
  for (int r = 0; r < PF; ++r) {
    const int c = c0 + r;
    if (c < nchunks) {
      commit(ring[(1 + r) % PF], c);
      lds_barrier();
      store(c - 1, true);      // not the last chunk
      compute(c);
    }
  }
  lds_barrier();
  store(nchunks - 1, nfull == nchunks);

  // X_t tiles of this wave's row tile: tile (ft, ct), lane's 4 values
  uint16_t* X = static_cast<uint16_t*>(a.X) + (((long)b * a.H + h0 + hp) * a.T + t) * DD +
                (ft * NT * 64 + lane) * 4;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    u32x2 pk;
    pk[0] = (uint32_t)f32_to_bf16_bits(acc[ct][0]) | ((uint32_t)f32_to_bf16_bits(acc[ct][1]) << 16);
    pk[1] = (uint32_t)f32_to_bf16_bits(acc[ct][2]) | ((uint32_t)f32_to_bf16_bits(acc[ct][3]) << 16);
    *reinterpret_cast<u32x2*>(X + ct * 256) = pk;
  }
}

template <int NT, bool CHAIN>
static void launch_xdq_chain(const XdqArgs& a, hipStream_t s) {
  if (a.H % 2 == 0)
    hipLaunchKernelGGL((xdq_kernel<NT, 2, CHAIN>), dim3(a.B * a.T * (a.H / 2)), dim3(128 * NT), 0,
                       s, a);
  else
    hipLaunchKernelGGL((xdq_kernel<NT, 1, CHAIN>), dim3(a.B * a.T * a.H), dim3(64 * NT), 0, s, a);
}
template <int NT>
static hipError_t launch_xdq_nt(const XdqArgs& a, hipStream_t s) {
  if (a.inv)
    launch_xdq_chain<NT, true>(a, s);
  else
    launch_xdq_chain<NT, false>(a, s);
  return hipGetLastError();
}

bool xdq_supported(int io, int64_t B, int64_t T, int64_t H) {
  return io == IO_BF16 && B * T * (H % 2 == 0 ? H / 2 : H) >= 256;
}

hipError_t launch_xdq(const XdqArgs& a, int io, int nt, hipStream_t s) {
  if (!xdq_supported(io, a.B, a.T, a.H)) return hipErrorNotSupported;
  switch (nt) {
    case 1: return launch_xdq_nt<1>(a, s);
    case 2: return launch_xdq_nt<2>(a, s);
    case 3: return launch_xdq_nt<3>(a, s);
    case 4: return launch_xdq_nt<4>(a, s);
    case 5: return launch_xdq_nt<5>(a, s);
    case 6: return launch_xdq_nt<6>(a, s);
    case 7: return launch_xdq_nt<7>(a, s);
    case 8: return launch_xdq_nt<8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
