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
// read S_0, so parts of kDirectPartTokens tokens are formed independently:
// one workgroup per (head, row block, part) takes the products of
// direct_kernel for its part (P = S_0 K^T, R = (s V^T - s^2 P) beta, dS_p =
// R K) and stores dS_p in fp32; direct_combine_kernel then sums the parts in
// a fixed order with the decay, S_1 = gamma S_0 + sum_p dS_p.  The
// per-workgroup chain of one chunk after another becomes one chunk plus the
// sum, and the launch fills the CUs (B H (D / 16) P workgroups).
template <int NT>
__global__ __launch_bounds__(64 * NT, 4) void direct_part_kernel(DirectArgs a) {
  typedef uint16_t E;                            // bf16 bits
  constexpr int D = 16 * NT;
  constexpr int KB = (D + 31) / 32;              // MFMA k blocks over the features
  constexpr int CK = kDirectPartTokens;          // tokens of a part
  constexpr int TT = CK / 16;                    // 16-token tiles
  constexpr int NW = NT;                         // waves
  constexpr int NTH = 64 * NW;
  constexpr int KPR = D * 2 / 16;                // 16-byte pieces per key row
  constexpr int KPC = CK * KPR;                  // key pieces of a part
  constexpr int KPT = (KPC + NTH - 1) / NTH;     // of them per thread
  constexpr int VPC = CK * 2;                    // 16-byte value pieces (16 features a token)
  constexpr int VPT = (VPC + NTH - 1) / NTH;
  constexpr int BPT = (CK + NTH - 1) / NTH;      // gates per thread
  constexpr int TPW = (TT + NW - 1) / NW;        // P tiles per wave
  constexpr int ZLD = D + 8;                     // staged state row (elements)
  constexpr int RLD = CK + 8;                    // staged R row (elements)
  static_assert(CK % 32 == 0, "whole 32-token MFMA blocks");
  static_assert(ZLD <= RLD, "the staged state rows fit the R buffer");
  // (the staged rows of S_0 share R's buffer: they are read into registers
  // before R is written, which keeps four workgroups per CU)
  __shared__ __attribute__((aligned(16))) E Ks[CK * D];
  __shared__ __attribute__((aligned(16))) E Rs[16 * RLD];
  E* const Zs = Rs;
  __shared__ __attribute__((aligned(16))) E Vs[CK * 16];          // values of the 16 rows
  __shared__ float bs[CK];                                        // gates of the tokens

  const int P = a.P;
  const int total = a.B * a.H * NT * P;
  const int item = xcd_item(blockIdx.x, total);  // a head's parts and row blocks share an XCD
  const int pt = item % P;
  const int rb = (item / P) % NT;
  const int bh = item / (P * NT);
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, H = a.H;
  const float s = a.s, s2 = a.s * a.s;
  const long DD = (long)D * D;
  const E* kp = static_cast<const E*>(a.k);
  const E* vp = static_cast<const E*>(a.v);
  const int n0 = pt * CK;
  // element (token n of frame 0, feature d): ((b T N + n) H + h) D + d
  auto rowbase = [&](int n) { return (((long)b * a.T) * N + n) * H + h; };

  // Every load in flight at once (clamped, never skipped: pieces past the
  // part's count re-read one inside it and are not committed; tokens past
  // the frame re-read its last row and get gate 0).
  u32x4 kr[KPT], vr[VPT];
  float br[BPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int q = min(tid + NTH * j, KPC - 1);
    const int n = min(n0 + q / KPR, N - 1);
    kr[j] = *reinterpret_cast<const u32x4*>(kp + rowbase(n) * D + (q % KPR) * 8);
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vt = min(tid + NTH * j, VPC - 1);
    const int n = min(n0 + vt / 2, N - 1);
    vr[j] = *reinterpret_cast<const u32x4*>(vp + rowbase(n) * D + rb * 16 + 8 * (vt % 2));
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int c = min(tid + NTH * j, CK - 1);
    br[j] = a.beta[rowbase(min(n0 + c, N - 1))];
  }
  // this lane's state: S_0[16 rb + 4 g + r][16 w + i]
  f32x4 z = zero4();
  if (a.z0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = a.z0[bh * DD + (rb * 16 + 4 * g + r) * D + w * 16 + li];
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) Zs[(4 * g + r) * ZLD + w * 16 + li] = f32_to_bf16_bits(z[r]);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int q = tid + NTH * j;
    if (q < KPC) *reinterpret_cast<u32x4*>(&Ks[(q / KPR) * D + (q % KPR) * 8]) = kr[j];
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vt = tid + NTH * j;
    if (vt < VPC) *reinterpret_cast<u32x4*>(&Vs[vt * 8]) = vr[j];
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int c = tid + NTH * j;
    if (c < CK) bs[c] = n0 + c < N ? br[j] : 0.f;
  }
  block_sync();

  // P = S_0[rows] K^T per 16-token tile, R = (s v - s^2 P) beta as [row][token]
  bf16x8 sz[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int k = kb * 32 + 8 * g;
    sz[kb] = k < D ? load_bf16x8(Zs + li * ZLD + k) : zero_bf16x8();
  }
  block_sync();   // every wave holds its rows of S_0 before R is written over them
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tt = w + NW * u;
    if (tt < TT) {
      f32x4 pr = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k = kb * 32 + 8 * g;
        const bf16x8 kf = k < D ? load_bf16x8(&Ks[(tt * 16 + li) * D + k]) : zero_bf16x8();
        pr = mfma_bf16(sz[kb], kf, pr);
      }
      const int tk = tt * 16 + li;
      const float bt = bs[tk];
      const u32x2 vv = *reinterpret_cast<const u32x2*>(&Vs[tk * 16 + 4 * g]);
      const float v4[4] = {bf16_bits_to_f32((uint16_t)(vv[0] & 0xffff)),
                           bf16_bits_to_f32((uint16_t)(vv[0] >> 16)),
                           bf16_bits_to_f32((uint16_t)(vv[1] & 0xffff)),
                           bf16_bits_to_f32((uint16_t)(vv[1] >> 16))};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Rs[(4 * g + r) * RLD + tk] = f32_to_bf16_bits((s * v4[r] - s2 * pr[r]) * bt);
    }
  }
  block_sync();

  // dS_p = R K on this wave's 16 features (keys by the transposing read)
  f32x4 dS = zero4();
#pragma unroll
  for (int kk = 0; kk < CK / 32; ++kk) {
    const bf16x8 rf = load_bf16x8(&Rs[li * RLD + kk * 32 + 8 * g]);
    const bf16x8 kf = lds_col_frag_bf16(Ks, D, kk * 32, w * 16);
    dS = mfma_bf16(rf, kf, dS);
  }
  *reinterpret_cast<f32x4*>(a.part + ((((long)bh * NT + rb) * P + pt) * NT + w) * 256 + lane * 4) =
      dS;
}

// S_1 = gamma S_0 + sum_p dS_p (parts in order), one lane of a part's tile
// layout per thread: fp32 to zT, bf16 to the emitted S_1.
template <int NT>
__global__ __launch_bounds__(256) void direct_combine_kernel(DirectArgs a) {
  constexpr int D = 16 * NT;
  const long DD = (long)D * D;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)a.B * a.H * NT * NT * 64) return;
  const int lane = (int)(e % 64);
  const int w = (int)((e / 64) % NT);
  const int rb = (int)((e / (64 * NT)) % NT);
  const long bh = e / (64 * NT * NT);
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int g = lane >> 4, li = lane & 15;
  const int P = a.P;
  const float* src = a.part + ((bh * NT + rb) * P * NT + w) * 256 + lane * 4;
  // the parts in order, eight loads in flight at a time
  f32x4 acc = zero4();
  for (int p0 = 0; p0 < P; p0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = *reinterpret_cast<const f32x4*>(src + (long)min(p0 + j, P - 1) * NT * 256);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j < P) acc += v[j];
  }
  const float gm = a.gamma[(long)b * a.T * a.H + h];
  uint16_t* Sout = static_cast<uint16_t*>(a.emit) + bh * a.T * DD;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const long idx = (rb * 16 + 4 * g + r) * D + w * 16 + li;
    const float z = gm * (a.z0 ? a.z0[bh * DD + idx] : 0.f) + acc[r];
    if (a.zT) a.zT[bh * DD + idx] = z;
    Sout[idx] = f32_to_bf16_bits(z);
  }
}

template <int NT>
static hipError_t launch_direct_split_nt(const DirectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((direct_part_kernel<NT>), dim3(a.B * a.H * NT * a.P), dim3(64 * NT), 0, s, a);
  const long lanes = (long)a.B * a.H * NT * NT * 64;
  hipLaunchKernelGGL((direct_combine_kernel<NT>), dim3((unsigned)((lanes + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_direct_split(const DirectArgs& a, int nt, hipStream_t s) {
  // one frame, parts covering its tokens with none empty
  if (a.T != 1 || a.N < 1 || a.P < 1 || !a.part || (long)a.P * kDirectPartTokens < a.N ||
      (long)(a.P - 1) * kDirectPartTokens >= a.N)
    return hipErrorInvalidValue;
  switch (nt) {
    case 1: return launch_direct_split_nt<1>(a, s);
    case 2: return launch_direct_split_nt<2>(a, s);
    case 3: return launch_direct_split_nt<3>(a, s);
    case 4: return launch_direct_split_nt<4>(a, s);
    case 5: return launch_direct_split_nt<5>(a, s);
    case 6: return launch_direct_split_nt<6>(a, s);
    case 7: return launch_direct_split_nt<7>(a, s);
    case 8: return launch_direct_split_nt<8>(a, s);
  }
  return hipErrorInvalidValue;
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
