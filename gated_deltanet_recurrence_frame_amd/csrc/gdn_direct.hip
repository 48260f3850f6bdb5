// Direct form of the frame-wise GDN state update for short launches
// (streaming steps, short windows): the frames are walked one after the
// other and every step works on the token rows themselves, with no
// per-frame D x D products.
//
// The module-2 update of the summary page (方法步骤详情), S_t = S_{t-1}
// (gamma_t I - K^_t beta_t K^_t^T) + V_t beta_t K^_t^T with K^ = s K, is,
// token by token of the frame (all of them read S_{t-1}),
//     S_t = gamma_t S_{t-1} + sum_n beta_n r_n k_n^T,
//     r_n = s v_n - s^2 S_{t-1} k_n.
// Rows of S evolve independently, so a workgroup owns 16 rows of one head's
// state (one wave per 16-column tile, the tile in fp32 registers).  Per
// frame it stages its rows of S_{t-1} in LDS (bf16) as MFMA operands, stores
// them as the previous frame's state, and streams the frame's keys in
// chunks of 128 tokens through LDS: per 16-token tile P = S_{t-1} K^T (keys
// read as rows), R = s V^T - s^2 P scaled by beta (values of its 16 rows
// read straight from memory), staged in LDS; then the update R K (keys read
// with the transposing LDS read) accumulates in every wave's tile.  The
// chunks of all frames form one sequence whose keys, values and gates ride
// in a register ring PK chunks ahead, across frame boundaries.  The states
// S_t go to the caller's buffer (bf16 row-major, as the scan emits them),
// from which the output kernel forms O_t = S_t Q_t for all frames at once.
// The same products as the frame form, with the state as one operand of
// each: one launch, sequential over frames, parallel over heads and row
// blocks.  It pays where the frame form's fixed costs (token splits of the
// Gram/write pass, their reduction, the scan launch) dominate: a handful
// of frames.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int NT>
__global__ __launch_bounds__(64 * NT) void direct_kernel(DirectArgs a) {
  typedef uint16_t E;                            // bf16 bits
  constexpr int D = 16 * NT;
  constexpr int KB = (D + 31) / 32;              // MFMA k blocks over the features
  constexpr int CK = 128;                        // tokens per chunk
  constexpr int TT = CK / 16;                    // 16-token tiles per chunk
  constexpr int NW = NT;                         // waves
  constexpr int NTH = 64 * NW;
  constexpr int KPR = D * 2 / 16;                // 16-byte pieces per key row
  constexpr int KPT = CK * KPR / NTH;            // of a chunk per thread
  constexpr int TPW = (TT + NW - 1) / NW;        // P tiles per wave
  constexpr int VPC = CK * 2;                    // 16-byte value pieces of a chunk
  constexpr int VPT = (VPC + NTH - 1) / NTH;     // of them per thread
  constexpr int BPT = (CK + NTH - 1) / NTH;      // gates per thread
  constexpr int ZLD = D + 8;                     // staged state row (elements)
  constexpr int RLD = CK + 8;                    // staged R row (elements)
  constexpr int PK = 3;                          // chunks in flight
  static_assert(KPT * NTH == CK * KPR, "key pieces split evenly");
  static_assert(16 * (D / 4) == NTH, "one 4-element piece of the staged rows per thread");
  __shared__ __attribute__((aligned(16))) E Kst[3][CK * D];
  __shared__ __attribute__((aligned(16))) E Rs[2][16 * RLD];
  __shared__ __attribute__((aligned(16))) E Zs[16 * ZLD];
  __shared__ __attribute__((aligned(16))) E Vs[3][CK * 16];       // values of the 16 rows
  __shared__ float bs[3][CK];                                     // gates of the tokens
  __shared__ float gs[3];                                         // the frame's decay

  const int total = a.B * a.H * NT;
  const int item = xcd_item(blockIdx.x, total);
  const int rb = item % NT;
  const int bh = item / NT;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, H = a.H, T = a.T;
  const float s = a.s, s2 = a.s * a.s;
  const long DD = (long)D * D;
  const E* kp = static_cast<const E*>(a.k);
  const E* vp = static_cast<const E*>(a.v);
  E* Sout = static_cast<E*>(a.emit) + (long)bh * T * DD;

  // this lane's state: S[16 rb + 4 g + r][16 w + i]
  f32x4 z = zero4();
  if (a.z0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = a.z0[bh * DD + (rb * 16 + 4 * g + r) * D + w * 16 + li];
  }

  const int nch = (N + CK - 1) / CK;
  const int nall = T * nch;                      // chunks of all frames
  // Ring slot: everything a chunk needs from memory, all of it committed to
  // LDS at once (a value kept in registers past the slot's reload would
  // have to be copied, and the copy would wait for every load in flight).
  struct Pre {
    u32x4 k[KPT];      // key pieces of the chunk
    u32x4 v[VPT];      // 8 of the 16 rows' values of one token each
    float bt[BPT];     // gates of tokens
    float gm;          // the frame's decay
  };
  // element (token n of frame t, feature d): (((b T + t) N + n) H + h) D + d
  auto rowbase = [&](int t, int n) { return (((long)b * T + t) * N + n) * H + h; };
  // loads clamped, never skipped (past the last chunk, past a frame's rows)
  auto prefetch = [&](Pre& P, int gc) {
    gc = gc < nall ? gc : nall - 1;
    const int t = gc / nch, c0 = (gc - t * nch) * CK;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int q = tid + NTH * j;
      int n = c0 + q / KPR;
      n = n < N ? n : N - 1;
      P.k[j] = *reinterpret_cast<const u32x4*>(kp + rowbase(t, n) * D + (q % KPR) * 8);
    }
    // (pieces past the chunk's count re-read one inside it and are not committed)
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vt = (tid + NTH * j) % VPC;
      int n = c0 + vt / 2;
      n = n < N ? n : N - 1;
      P.v[j] = *reinterpret_cast<const u32x4*>(vp + rowbase(t, n) * D + rb * 16 + 8 * (vt % 2));
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      int n = c0 + (tid + NTH * j) % CK;
      n = n < N ? n : N - 1;
      P.bt[j] = a.beta[rowbase(t, n)];
    }
    P.gm = a.gamma[((long)b * T + t) * H + h];
  };
  auto stage_z = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) Zs[(4 * g + r) * ZLD + w * 16 + li] = f32_to_bf16_bits(z[r]);
  };
  auto emit_rows = [&](int t) {   // the staged rows as S_t
    constexpr int PRW = D / 4;
    const int row = tid / PRW, pc = tid % PRW;
    *reinterpret_cast<u32x2*>(Sout + t * DD + (rb * 16 + row) * D + pc * 4) =
        *reinterpret_cast<const u32x2*>(&Zs[row * ZLD + pc * 4]);
  };

  bf16x8 sz[KB];   // this block's rows of S_{t-1}, left operand of P
  f32x4 dS = zero4();
  auto load_sz = [&]() {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 32 + 8 * g;
      sz[kb] = load_bf16x8(Zs + li * ZLD + (k < D ? k : 0));
      if (k >= D) sz[kb] = zero_bf16x8();
    }
  };
  // chunk gc's keys, values, gates and decay into LDS buffer gc % 3
  auto commit = [&](const Pre& R, int gc) {
    const int sk = gc % 3;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int q = tid + NTH * j;
      *reinterpret_cast<u32x4*>(&Kst[sk][(q / KPR) * D + (q % KPR) * 8]) = R.k[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      if (tid + NTH * j < VPC) *reinterpret_cast<u32x4*>(&Vs[sk][(tid + NTH * j) * 8]) = R.v[j];
#pragma unroll
    for (int j = 0; j < BPT; ++j)
      if (tid + NTH * j < CK) bs[sk][tid + NTH * j] = R.bt[j];
    if (tid == 0) gs[sk] = R.gm;
  };
  // P = S K^T per 16-token tile of chunk gc, R = (s v - s^2 P) beta staged
  // as [row][token] in R buffer gc % 2
  auto compute_p = [&](int gc) {
    const int sk = gc % 3, sr = gc & 1;
    const int c = gc % nch;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + NW * u;
      if (tt < TT) {
        f32x4 p = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int k = kb * 32 + 8 * g;
          bf16x8 kf = load_bf16x8(&Kst[sk][(tt * 16 + li) * D + (k < D ? k : 0)]);
          if (k >= D) kf = zero_bf16x8();
          p = mfma_bf16(sz[kb], kf, p);
        }
        // tokens past the frame's end (re-read rows) write nothing
        const int tk = tt * 16 + li;
        const float bt = (c * CK + tk < N) ? bs[sk][tk] : 0.f;
        const u32x2 vv = *reinterpret_cast<const u32x2*>(&Vs[sk][tk * 16 + 4 * g]);
        const float v4[4] = {bf16_bits_to_f32((uint16_t)(vv[0] & 0xffff)),
                             bf16_bits_to_f32((uint16_t)(vv[0] >> 16)),
                             bf16_bits_to_f32((uint16_t)(vv[1] & 0xffff)),
                             bf16_bits_to_f32((uint16_t)(vv[1] >> 16))};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Rs[sr][(4 * g + r) * RLD + tk] = f32_to_bf16_bits((s * v4[r] - s2 * p[r]) * bt);
      }
    }
  };
  // the update of this wave's tile by chunk gc: R (rows x tokens) times K
  // (tokens x 16 features)
  auto compute_ds = [&](int gc) {
    const int sk = gc % 3, sr = gc & 1;
#pragma unroll
    for (int kk = 0; kk < CK / 32; ++kk) {
      const bf16x8 rf = load_bf16x8(&Rs[sr][li * RLD + kk * 32 + 8 * g]);
      const bf16x8 kf = lds_col_frag_bf16(&Kst[sk][0], D, kk * 32, w * 16);
      dS = mfma_bf16(rf, kf, dS);
    }
  };

  // Software pipeline, one barrier per chunk: step i commits chunk i + 1
  // (and reloads its ring slot PK chunks ahead), then computes P of chunk
  // i + 1 next to the update by chunk i (K in three LDS buffers, R in two).
  // At a frame's last chunk the state is updated, staged and P of the next
  // frame's first chunk follows behind one more barrier.  The staged rows
  // are stored as the previous frame's state at every step (the same bytes
  // each time: a store under a branch would cost the compiler its count of
  // the loads in flight; frame 0 stores S_{-1} into slot 0, which S_0
  // overwrites later).
  auto step = [&](Pre& R, int i) {
    const int t = i / nch, c = i - t * nch;
    commit(R, i + 1);
    prefetch(R, i + 1 + PK);
    emit_rows(t > 0 ? t - 1 : 0);
    lds_barrier();
    const bool last = c == nch - 1;
    if (!last && i + 1 < nall) compute_p(i + 1);
    compute_ds(i);
    if (last) {
      z = gs[i % 3] * z + dS;
      dS = zero4();
      if (i + 1 < nall) {
        stage_z();
        lds_barrier();
        load_sz();
        compute_p(i + 1);
      }
    }
  };

  Pre ring[PK];
#pragma unroll
  for (int r = 0; r < PK; ++r) prefetch(ring[r], r);
  stage_z();
  lds_barrier();
  load_sz();
  commit(ring[0], 0);
  prefetch(ring[0], PK);
  lds_barrier();
  compute_p(0);
  // whole trips of PK steps straight-line (no branch around a memory
  // operation), then the last, partial trip; step i uses ring slot i + 1
  int i0 = 0;
  for (; i0 + PK <= nall; i0 += PK) {
#pragma unroll
    for (int r = 0; r < PK; ++r) step(ring[(r + 1) % PK], i0 + r);
  }
#pragma unroll
  for (int r = 0; r < PK; ++r)
    if (i0 + r < nall) step(ring[(r + 1) % PK], i0 + r);
  // the last frame's state
  lds_barrier();
  stage_z();
  lds_barrier();
  emit_rows(T - 1);
  if (a.zT) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a.zT[bh * DD + (rb * 16 + 4 * g + r) * D + w * 16 + li] = z[r];
  }
}

// One frame with its tokens split over parts (streaming steps of many
// tokens).  The update of a frame is a sum over its tokens, all of which
// read S_0, so parts of kDirectPartTokens tokens are formed independently,
// and the rows of S evolve independently, so the output features of a row
// block need only those rows of S_1.  Two launches:
//
// direct_part_kernel, one workgroup per (head, part), one wave per 16-row
// block of the state.  The part's key and value rows are staged in LDS once
// for all row blocks.  Each wave forms, for its rows r0 .. r0 + 15,
//   P^T = K S_0[rows]^T            (tokens x rows; MFMA with the key rows as
//                                   the left operand and its rows of S_0,
//                                   rounded to bf16, as the right one)
//   R^T = (s V[:, rows] - s^2 P^T) beta     (fp32, rounded to bf16)
//   dS_p[rows]^T = K^T R^T         (features x rows)
// The accumulator tiles of R^T give each lane, for its row, the tokens
// 4 g .. + 3 and 16 + 4 g .. + 3 of each 32-token block: the second
// product takes that token order in both operands (the keys' columns by two
// transposing LDS reads of 4 rows each), so R never leaves the registers.
// dS_p is stored as transposed tiles (lane (g, i) of tile j holds
// dS_p[r0 + i][16 j + 4 g .. + 3]) in fp32.
//
// direct_out_kernel, one workgroup per (head, row block): its waves sum the
// parts in a fixed order with the decay, S_1 = gamma S_0 + sum_p dS_p (one
// tile per wave; fp32 rows to the state, bf16 rows through LDS to every
// wave), then form the output features r0 .. r0 + 15 of every token,
// O[n][rows] = S_1[rows] q_n: the rounded rows of S_1 are the left operand,
// the query rows the right one, read straight from memory as 16-byte
// pieces (8-byte pieces in the tiles' feature order made every load touch
// 16 lines for 32 bytes each, and the kernel about a third slower).  Each
// lane stores 4 contiguous output features of one token.
template <int NT>
__global__ __launch_bounds__(64 * NT) void direct_part_kernel(DirectArgs a) {
  typedef uint16_t E;                            // bf16 bits
  constexpr int D = 16 * NT;
  constexpr int KF = D / 32;                     // full 32-feature blocks
  constexpr bool HALF = (D % 32) == 16;          // a last block of 16 features
  constexpr int KB = KF + (HALF ? 1 : 0);
  constexpr int CK = kDirectPartTokens;          // tokens of a part
  constexpr int TT = CK / 16;                    // 16-token tiles
  constexpr int TB = CK / 32;                    // 32-token blocks
  constexpr int NTH = 64 * NT;
  constexpr int PRW = D * 2 / 16;                // 16-byte pieces per row
  constexpr int RPC = CK * PRW;                  // pieces of the part's key (or value) rows
  constexpr int PPT = (RPC + NTH - 1) / NTH;     // of them per thread
  constexpr int LDK = D + 8;                     // staged row (elements; a 16-byte multiple)
  constexpr int BPT = (CK + NTH - 1) / NTH;      // gates per thread
  static_assert(CK % 32 == 0, "whole 32-token blocks");
  __shared__ __attribute__((aligned(16))) E Ks[CK * LDK];
  __shared__ __attribute__((aligned(16))) E Vs[CK * LDK];
  __shared__ __attribute__((aligned(16))) float bs[CK];

  const int P = a.P;
  const int total = a.B * a.H * P;
  const int item = xcd_item(blockIdx.x, total);  // a head's parts share an XCD
  const int pt = item % P;
  const int bh = item / P;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), rb = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, H = a.H;
  const float s = a.s, s2 = a.s * a.s;
  const long DD = (long)D * D;
  const E* kp = static_cast<const E*>(a.k);
  const E* vp = static_cast<const E*>(a.v);
  const int n0 = pt * CK;
  // element (token n of the frame, feature d): ((b N + n) H + h) D + d  (T == 1)
  auto rowbase = [&](int n) { return (((long)b * N + n) * H + h) * D; };

  // Every load in flight at once (clamped, never skipped: pieces past the
  // count re-read the last one and are not committed; tokens past the frame
  // re-read its last row and get gate 0, so they add exact zeros).
  u32x4 kr[PPT], vr[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int q = min(tid + NTH * j, RPC - 1);
    const long off = rowbase(min(n0 + q / PRW, N - 1)) + (q % PRW) * 8;
    kr[j] = *reinterpret_cast<const u32x4*>(kp + off);
    vr[j] = *reinterpret_cast<const u32x4*>(vp + off);
  }
  float bt[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    bt[j] = a.beta[((long)b * N + min(n0 + min(tid + NTH * j, CK - 1), N - 1)) * H + h];
  // this wave's rows of S_0 as the right operand: lane (g, i) holds
  // S_0[r0 + i][32 kb + 8 g .. + 7] (features past D zero)
  bf16x8 sz[KB];
  {
    const float* zr = a.z0 ? a.z0 + bh * DD + (long)(rb * 16 + li) * D : nullptr;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int f = kb * 32 + 8 * g;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (zr) {   // uniform; lanes past D re-read an inside piece and zero it
        const int fc = min(f, D - 8);
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(zr + fc);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(zr + fc + 4);
        const float m = f < D ? 1.f : 0.f;
        v[0] = m * a0[0]; v[1] = m * a0[1]; v[2] = m * a0[2]; v[3] = m * a0[3];
        v[4] = m * a1[0]; v[5] = m * a1[1]; v[6] = m * a1[2]; v[7] = m * a1[3];
      }
      sz[kb] = f32x8_to_bf16x8(v);
    }
  }
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int q = tid + NTH * j;
    if (RPC % NTH == 0 || q < RPC) {
      *reinterpret_cast<u32x4*>(&Ks[(q / PRW) * LDK + (q % PRW) * 8]) = kr[j];
      *reinterpret_cast<u32x4*>(&Vs[(q / PRW) * LDK + (q % PRW) * 8]) = vr[j];
    }
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int c = tid + NTH * j;
    if (c < CK) bs[c] = n0 + c < N ? bt[j] : 0.f;
  }
  block_sync();

  // R^T tiles: lane (g, i) of tile t holds R[r0 + i][16 t + 4 g + j], j = 0..3
  u32x2 rt[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    f32x4 pr = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int f = kb * 32 + 8 * g;
      // (lanes past D: their S_0 operand is zero, so any finite keys add 0)
      const bf16x8 kf = load_bf16x8(&Ks[(t * 16 + li) * LDK + min(f, D - 8)]);
      pr = mfma_bf16(kf, sz[kb], pr);
    }
    const i16x4 vv = lds_rows4_tr(Vs, LDK, t * 16 + 4 * g, rb * 16);
    const f32x4 bb = *reinterpret_cast<const f32x4*>(&bs[t * 16 + 4 * g]);
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (s * bf16_bits_to_f32((uint16_t)vv[j]) - s2 * pr[j]) * bb[j];
    rt[t] = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[0], r[1]}, bf16x2)),
                  __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[2], r[3]}, bf16x2))};
  }
  // dS_p^T tiles: K^T (features x tokens) times R^T (tokens x rows), the
  // tokens of block tb in the order of the R^T tiles 2 tb, 2 tb + 1
  float* out = a.part + (((long)bh * NT + rb) * P + pt) * NT * 256 + lane * 4;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    f32x4 acc = zero4();
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const i16x4 k0 = lds_rows4_tr(Ks, LDK, tb * 32 + 4 * g, jt * 16);
      const i16x4 k1 = lds_rows4_tr(Ks, LDK, tb * 32 + 16 + 4 * g, jt * 16);
      const bf16x8 kc = __builtin_bit_cast(bf16x8, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
      const u32x2 lo = rt[2 * tb], hi = rt[2 * tb + 1];
      acc = mfma_bf16(kc, __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]}), acc);
    }
    *reinterpret_cast<f32x4*>(out + jt * 256) = acc;
  }
}

// S_1 = gamma S_0 + sum_p dS_p (parts in order) for the rows of one row
// block, then the output features of those rows for every token.
constexpr int kDirectOutWaves = 16;
template <int NT>
__global__ __launch_bounds__(64 * kDirectOutWaves) void direct_out_kernel(DirectArgs a) {
  typedef uint16_t E;
  constexpr int D = 16 * NT;
  constexpr int KF = D / 32;
  constexpr bool HALF = (D % 32) == 16;
  constexpr int KB = KF + (HALF ? 1 : 0);
  constexpr int NW = kDirectOutWaves;            // waves
  constexpr int UT = 4;                          // token tiles of a wave in flight at once
  constexpr int SLD = D + 8;                     // staged row (elements)
  static_assert(NT <= NW, "one wave per tile of the row block's sum");
  __shared__ __attribute__((aligned(16))) uint16_t s1r[16 * SLD];   // rounded S_1 rows

  const int total = a.B * a.H * NT;
  const int item = xcd_item(blockIdx.x, total);  // a head's row blocks share an XCD
  const int rb = item % NT;
  const int bh = item / NT;
  const int b = bh / a.H, h = bh % a.H;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, H = a.H, P = a.P;
  const long DD = (long)D * D;
  const float gm = a.gamma[(long)b * H + h];     // T == 1

  // O[n][r0 + 4 g + r] for the tokens n = 16 t + i of this wave's tiles
  // t = w + NW u, UT tiles at a time with all their query loads in flight
  // (clamped to the frame's last row, stores only for tokens inside it).
  // The queries do not depend on S_1: the first tiles' loads are issued
  // before the parts', so the two latencies overlap.
  const E* qp = static_cast<const E*>(a.q);
  E* op = static_cast<E*>(a.o);
  const int TQ = (N + 15) / 16;
  bf16x8 qf[UT][KB];
  auto load_q = [&](int t0) {
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int n = (t0 + NW * u) * 16 + li;
      const long row = (((long)b * N + min(n, N - 1)) * H + h) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // unconditional (a branch around a load makes the compiler wait for
        // every load in flight where the paths join): lanes past D re-read
        // an inside piece of the row and zero it
        const int f = kb * 32 + 8 * g;
        const bf16x8 v = load_bf16x8(qp + row + min(f, D - 8));
        qf[u][kb] = f < D ? v : zero_bf16x8();
      }
    }
  };
  load_q(w);

  // S_1 rows r0 + i, features 16 j + 4 g .. + 3 (transposed tile j), tile j
  // by wave j.  Each element is read (S_0) and written (the state, which may
  // be S_0 itself) by the same lane only.
  if (w < NT) {
    const int j = w;
    const long zoff = bh * DD + (long)(rb * 16 + li) * D + 4 * g + 16 * j;
    const float* src = a.part + (((long)bh * NT + rb) * P * NT + j) * 256 + lane * 4;
    f32x4 acc = a.z0 ? gm * *reinterpret_cast<const f32x4*>(a.z0 + zoff) : zero4();
    for (int p0 = 0; p0 < P; p0 += 8) {   // the parts in order, eight loads in flight
      f32x4 v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        v[c] = *reinterpret_cast<const f32x4*>(src + (long)min(p0 + c, P - 1) * NT * 256);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (p0 + c < P) acc += v[c];
    }
    if (a.zT) *reinterpret_cast<f32x4*>(a.zT + zoff) = acc;
    *reinterpret_cast<u32x2*>(&s1r[li * SLD + 16 * j + 4 * g]) =
        u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{acc[0], acc[1]}, bf16x2)),
              __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{acc[2], acc[3]}, bf16x2))};
  }
  block_sync();
  // left operand: S_1[r0 + i][32 kb + 8 g .. + 7] (features past D zero)
  bf16x8 sa[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int f = kb * 32 + 8 * g;
    const bf16x8 v = load_bf16x8(&s1r[li * SLD + min(f, D - 8)]);
    sa[kb] = f < D ? v : zero_bf16x8();
  }
  for (int t0 = w; t0 < TQ; t0 += NW * UT) {
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mfma_bf16(sa[kb], qf[u][kb], acc);
      const int n = (t0 + NW * u) * 16 + li;
      // non-temporal: the outputs are not read again here
      if (n < N)
        __builtin_nontemporal_store(
            u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{acc[0], acc[1]}, bf16x2)),
                  __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{acc[2], acc[3]}, bf16x2))},
            reinterpret_cast<u32x2*>(op + (((long)b * N + n) * H + h) * D + rb * 16 + 4 * g));
    }
    if (t0 + NW * UT < TQ) load_q(t0 + NW * UT);
  }
}

template <int NT>
static hipError_t launch_direct_split_nt(const DirectArgs& a, bool out, hipStream_t s) {
  if (!out)
    hipLaunchKernelGGL((direct_part_kernel<NT>), dim3(a.B * a.H * a.P), dim3(64 * NT), 0, s, a);
  else
    hipLaunchKernelGGL((direct_out_kernel<NT>), dim3(a.B * a.H * NT), dim3(64 * kDirectOutWaves), 0,
                       s, a);
  return hipGetLastError();
}

static hipError_t launch_direct_split_any(const DirectArgs& a, int nt, bool out, hipStream_t s) {
  // one frame, parts covering its tokens with none empty
  if (a.T != 1 || a.N < 1 || a.P < 1 || !a.part || (long)a.P * kDirectPartTokens < a.N ||
      (long)(a.P - 1) * kDirectPartTokens >= a.N || (out && (!a.q || !a.o)))
    return hipErrorInvalidValue;
  switch (nt) {
    case 1: return launch_direct_split_nt<1>(a, out, s);
    case 2: return launch_direct_split_nt<2>(a, out, s);
    case 3: return launch_direct_split_nt<3>(a, out, s);
    case 4: return launch_direct_split_nt<4>(a, out, s);
    case 5: return launch_direct_split_nt<5>(a, out, s);
    case 6: return launch_direct_split_nt<6>(a, out, s);
    case 7: return launch_direct_split_nt<7>(a, out, s);
    case 8: return launch_direct_split_nt<8>(a, out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_direct_parts(const DirectArgs& a, int nt, hipStream_t s) {
  return launch_direct_split_any(a, nt, false, s);
}
hipError_t launch_direct_out(const DirectArgs& a, int nt, hipStream_t s) {
  return launch_direct_split_any(a, nt, true, s);
}

template <int NT>
static hipError_t launch_direct_nt(const DirectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((direct_kernel<NT>), dim3(a.B * a.H * NT), dim3(64 * NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_direct(const DirectArgs& a, int nt, hipStream_t s) {
  if (a.T < 1 || a.N < 1) return hipErrorInvalidValue;
  switch (nt) {
    case 1: return launch_direct_nt<1>(a, s);
    case 2: return launch_direct_nt<2>(a, s);
    case 3: return launch_direct_nt<3>(a, s);
    case 4: return launch_direct_nt<4>(a, s);
    case 5: return launch_direct_nt<5>(a, s);
    case 6: return launch_direct_nt<6>(a, s);
    case 7: return launch_direct_nt<7>(a, s);
    case 8: return launch_direct_nt<8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
