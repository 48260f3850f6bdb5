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
// Layout of the work: one workgroup per (b, t) frame and pair of adjacent
// heads (one per CU) when H is even, else per single head (two per CU); a
// head's row tiles are shared by up to 8 waves, one tile each when there
// are 5 to 8 tiles (head dims 80 to 128).  XCD-aware ordering
// so the heads of one frame run together on one XCD.  Tokens stream through
// LDS in chunks of CT rows (natural [token][feature] layout, the head
// group's row segments side by side, double-buffered); each thread loads
// two 16-byte pieces of every chunk into a register ring PF chunks ahead,
// with ordinary loads whose waits the compiler tracks, and commits them to
// LDS one chunk at a time behind an LDS-only barrier, so the ring stays in
// flight across it.  (Direct-to-LDS copies move the same bytes, but at
// this number of waves per CU they ran about a tenth slower.)
// The token rows are loaded non-temporally: they stream through once, and
// the caches keep the A_t and U_t just written for the scan that reads them
// next (the scan took 80 instead of 58 us at the one-minute shape when the
// rows went through the caches).
// Both MFMA operands need a feature's values over consecutive tokens; they
// are read with the gfx950 transposing LDS read.  The weight w multiplies
// the X operand in fp32 before rounding to bf16.  Tail tokens of the last
// chunk re-read the frame's last row and get weight 0, so they add exactly 0.
// Normalised keys (NORM, forward only): K^ = s K / |K| per token row,
// normalised on the way into LDS, no pass over K of its own.  The key
// pieces are then dealt by whole head rows, one DPP row of 16 lanes per
// row (two for fp32 rows of more than 16 pieces): each lane sums the
// squares of its piece, the row's lanes add them up, and every lane
// scales its piece by 1 / |k| before committing it; the products then run
// on the normalised keys exactly as without NORM.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Waves per head: one per 16-row tile of the products from 5 tiles up (no
// wave repeats another's tile), else 8 (the smaller heads' tiles repeated).
// NORM deals a chunk's key rows 16 lanes a row and keeps 8.
constexpr int gram_wph(int nt, bool norm) { return (nt >= 5 && !norm) ? nt : 8; }

template <int IO, int NT, int NR, bool Y_IS_X0, int HPW, bool NORM>
struct GramCfg {
  static constexpr bool BF = (IO == IO_BF16);
  static constexpr int D = 16 * NT;
  static constexpr int ES = Io<IO>::bytes;
  static constexpr int WPH = gram_wph(NT, NORM);            // waves per head
  static constexpr int NW = WPH * HPW;                      // waves
  static constexpr int NTH = 64 * NW;
  static constexpr int RW = HPW * D;                        // elements of a token's row segment
  static constexpr int CT = BF ? 32 : 16;                   // tokens per chunk
  static constexpr int NMAT = NR + (Y_IS_X0 ? 0 : 1);       // matrices staged
  static constexpr int PR = RW * ES / 16;                   // 16-byte pieces per row segment
  static constexpr int MPC = CT * PR;                       // pieces per matrix per chunk
  static constexpr int PPM = (MPC + NTH - 1) / NTH;         // of them per thread
  static constexpr int PPT = NMAT * PPM;                    // pieces per thread
  static constexpr int NWT = CT * HPW;                      // weights per chunk
  static constexpr int PH = D * ES / 16;                    // 16-byte pieces per head row
  // NORM: key pieces by head rows, LPR lanes a row (pieces past PH idle)
  static constexpr int LPR = PH <= 16 ? 16 : 32;
  static constexpr int NK = CT * HPW * LPR;                 // lanes dealt key pieces
  // LDS row stride (elements).  A fragment read takes the same 16 bf16 (or
  // 16 fp32) columns of 4 consecutive token rows per group of lanes; rows
  // are padded so that those rows start on different banks of the 32
  // (stride = 8 or 24 dwords mod 32 for bf16, 16 mod 32 for fp32).
  static constexpr int pad_for(int rw) {
    for (int p = 0; p < 64; p += (BF ? 8 : 4)) {
      const int sd = (rw + p) * ES / 4;
      if (BF ? (sd % 32 == 8 || sd % 32 == 24) : (sd % 32 == 16)) return p;
    }
    return 0;
  }
  static constexpr int LDR = RW + pad_for(RW);
  static constexpr int STAGE_ELEMS = NMAT * CT * LDR;
  static constexpr int PF = 2;                              // chunks in flight
  static constexpr int RPM = (NT + WPH - 1) / WPH;          // row tiles per wave per matrix
  static constexpr int RT = NR * RPM;                       // row tiles per wave
  static_assert(NWT <= NTH, "one weight per thread at most");
};

// Work item v (0 <= v < total) of a launch: frame (b, t), head group, token split.
struct GramItem {
  long row0;     // first token row of the frame
  int b, tl, h0, sp;
  int cbeg;      // first chunk of the split
  int n;         // chunks of the split (may be 0)
};

// SPLIT: the launch splits frames' tokens (a.P > 1) and stores fp32
// partials; a compile-time choice, so that no branch joins stores of the two
// kinds (the compiler would lose its count of the stores in flight).
template <int IO, int NT, int NR, bool Y_IS_X0, int HPW, bool SPLIT, bool NORM>
__global__ __launch_bounds__(64 * gram_wph(NT, NORM) * HPW, HPW == 1 ? 2 : 1) void gram_kernel(
    GramArgs a) {
  typedef GramCfg<IO, NT, NR, Y_IS_X0, HPW, NORM> C;
  static_assert(!NORM || (NR == 2 && Y_IS_X0), "normalised keys: X_0 == Y == K, X_1 == V");
  static_assert(!NORM || (C::NK <= C::NTH && C::PPM == 1), "one key piece per thread");
  typedef typename Io<IO>::elem E;
  constexpr int D = C::D, CT = C::CT, ES = C::ES, PR = C::PR, NTH = C::NTH;
  constexpr int LDR = C::LDR;
  __shared__ __attribute__((aligned(16))) E stage[2][C::STAGE_ELEMS];
  __shared__ float wstage[2][C::NWT];

  const int HG = a.H / HPW;                        // head groups
  const int total = a.B * a.Tc * HG * a.P;
  const int N = a.N;
  const int nchunks_all = (N + CT - 1) / CT;
  const int cps = (nchunks_all + a.P - 1) / a.P;  // chunks per split
  constexpr int PF = C::PF;
  const int ncp = (cps + PF - 1) / PF * PF;        // ring steps per item (whole trips)
  auto decode = [&](int v) {
    GramItem it;
    const int item = xcd_item(v, total);
    it.sp = item % a.P;
    it.h0 = ((item / a.P) % HG) * HPW;
    it.tl = (item / (a.P * HG)) % a.Tc;
    it.b = item / (a.P * HG * a.Tc);
    it.row0 = (long)it.b * a.T * N + (long)(a.t0 + it.tl) * N;
    it.cbeg = it.sp * cps;
    const int n = min(nchunks_all, it.cbeg + cps) - it.cbeg;
    it.n = n > 0 ? n : 0;
    return it;
  };

  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int hp = wave / C::WPH, wl = wave % C::WPH;   // this wave's head (in the group), slot
  const int g = lane >> 4, li = lane & 15;

  // staged matrix m: X_0, then X_1 (NR == 2) or Y (NR == 1, Y distinct)
  const E* src0 = static_cast<const E*>(a.x0);
  const E* src1 = static_cast<const E*>(NR == 2 ? a.x1 : a.y);
  const bool has_w = a.w != nullptr;

  // Register ring: chunk c of an item: pieces q = tid + NTH j of each
  // staged matrix ([CT][row segment], rows LDR apart in LDS) and one weight
  // ([token][head] of the group).  (NORM: the keys' piece of thread tid is
  // piece tid % LPR of head (tid / LPR) % HPW of token tid / (HPW LPR).)  Loads are clamped, never skipped (past
  // the item's last chunk, past the frame's last row, past the matrix's
  // last piece), so the loop stays straight-line and the compiler's wait
  // counts exact.  Addresses are a uniform 64-bit frame base plus 32-bit
  // per-lane offsets from 24-bit multiplies (the host keeps a frame's rows
  // under 2 GiB and N, H D es under 2^24), a few full-rate instructions
  // per piece.
  struct Ring {
    u32x4 v[C::PPT];
    float w;
  };
  const unsigned rowb = (unsigned)(a.H * D * ES);     // bytes between tokens
  auto load = [&](Ring& R, const GramItem& it, int c) {
    const int cl = it.n > 0 ? (c < it.n ? c : it.n - 1) : 0;
    const int c0 = (it.n > 0 ? it.cbeg + cl : 0) * CT;
    const long fb = (it.row0 * a.H + it.h0) * (long)(D * ES);
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m) {
      const char* base = reinterpret_cast<const char*>(m == 0 ? src0 : src1) + fb;
#pragma unroll
      for (int j = 0; j < C::PPM; ++j) {
        int q = tid + NTH * j;
        if (C::MPC % NTH != 0) q = q < C::MPC ? q : C::MPC - 1;
        int row = q / PR, col = q % PR;
        if (NORM && m == 0) {
          row = min(tid / (HPW * C::LPR), CT - 1);
          col = ((tid / C::LPR) % HPW) * C::PH + min(tid % C::LPR, C::PH - 1);
        }
        int tk = c0 + row;
        tk = tk < N ? tk : N - 1;
        const unsigned off = __umul24((unsigned)tk, rowb) + (unsigned)(col * 16);
        R.v[m * C::PPM + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
      }
    }
    // the first NWT threads load the chunk's weights; the others load one
    // shared address (a single cache line)
    // (without weights: a dummy load of the first input, value unused)
    const int wi = tid < C::NWT ? tid : 0;
    int tk = c0 + wi / HPW;
    tk = tk < N ? tk : N - 1;
    const float* wb = has_w ? a.w + it.row0 * a.H + it.h0 : reinterpret_cast<const float*>(src0);
    const unsigned woff = has_w ? __umul24((unsigned)tk, (unsigned)a.H) + (unsigned)(wi % HPW) : 0u;
    R.w = wb[woff];
  };
  auto commit = [&](const Ring& R, int st, int nv) {   // nv: tokens of the chunk in the frame
#pragma unroll
    for (int m = NORM ? 1 : 0; m < C::NMAT; ++m)
#pragma unroll
      for (int j = 0; j < C::PPM; ++j) {
        const int q = tid + NTH * j;
        if (C::MPC % NTH == 0 || q < C::MPC)
          *reinterpret_cast<u32x4*>(&stage[st][(m * CT + q / PR) * LDR + (q % PR) * (16 / ES)]) =
              R.v[m * C::PPM + j];
      }
    if constexpr (NORM) {   // the keys, by head rows
      const int row = tid / (HPW * C::LPR), pc = tid % C::LPR;
      const int col = ((tid / C::LPR) % HPW) * C::PH + pc;
      const float live = (row < CT && pc < C::PH) ? 1.f : 0.f;   // from tid only
      u32x4 v = R.v[0];
      float ss = live * piece_sumsq<IO>(v);
      ss = row_sum16(ss);
      if constexpr (C::LPR == 32) ss += __shfl_xor(ss, 16);
      v = piece_scale<IO>(v, inv_norm(ss));
      if (row < CT && pc < C::PH)
        *reinterpret_cast<u32x4*>(&stage[st][row * LDR + col * (16 / ES)]) = v;
    }
    // tokens past the frame's end get weight 0 (their rows are re-read copies)
    if (tid < C::NWT) wstage[st][tid] = tid / HPW < nv ? (has_w ? R.w : 1.0f) : 0.0f;
  };

  f32x4 acc[C::RT][NT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int j = 0; j < C::RT; ++j)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) acc[j][ct] = zero4();
  };

  auto compute = [&](int st) {
    // this wave's head: its D features at offset hp * D of each row segment
    const E* xs = &stage[st][hp * D];
    const E* ys = Y_IS_X0 ? xs : xs + (C::NMAT - 1) * CT * LDR;
    const float* ws = wstage[st];
    if constexpr (C::BF) {
      float wv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = ws[(8 * g + e) * HPW + hp];
      // the wave's weighted row fragments first, then one column fragment at
      // a time (few fragments live next to the accumulators)
      bf16x8 af[C::RT];
#pragma unroll
      for (int j = 0; j < C::RT; ++j) {
        // row tile j of every wave: matrix m = j / RPM, tile ft = wl + WPH
        // (j % RPM); every wave runs all RT (no branch in the loop), one past
        // NT repeats tile NT - 1 and is dropped at the end
        const int m = j / C::RPM;
        const int ft = min(wl + C::WPH * (j % C::RPM), NT - 1);
        af[j] = lds_col_frag_bf16(reinterpret_cast<const uint16_t*>(xs + m * CT * LDR), LDR, 0,
                                  ft * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          af[j][e] = static_cast<__bf16>(static_cast<float>(af[j][e]) * wv[e]);
      }
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const bf16x8 bfr = lds_col_frag_bf16(reinterpret_cast<const uint16_t*>(ys), LDR, 0, ct * 16);
#pragma unroll
        for (int j = 0; j < C::RT; ++j) acc[j][ct] = mfma_bf16(af[j], bfr, acc[j][ct]);
      }
    } else {
      // not unrolled: hoisting every k step's operands would spill
#pragma unroll 1
      for (int kb = 0; kb < CT / 4; ++kb) {
        const int k = kb * 4 + g;
        const float wv = ws[k * HPW + hp];
        float bfr[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) bfr[ct] = reinterpret_cast<const float*>(ys)[k * LDR + ct * 16 + li];
#pragma unroll
        for (int j = 0; j < C::RT; ++j) {
          const int m = j / C::RPM;   // see the bf16 path
          const int ft = min(wl + C::WPH * (j % C::RPM), NT - 1);
          const float af =
              reinterpret_cast<const float*>(xs + m * CT * LDR)[k * LDR + ft * 16 + li] * wv;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) acc[j][ct] = mfma_f32(af, bfr[ct], acc[j][ct]);
        }
      }
    }
  };

  // Results of an item straight from the accumulators (C[m][n] in lane
  // (g, n) register r with m = 4g + r): fp32 partial sums (token splits),
  // the tiles layout (4 contiguous values per lane), or a row-major matrix,
  // requested only for symmetric products (A_t): tile (I, J) read by
  // columns is row pieces of tile (J, I), 4 contiguous values of one row
  // per lane.
  auto pack = [&](const f32x4& v, E* dst) {
    if constexpr (C::BF) {
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
      *reinterpret_cast<f32x4*>(dst) = v;
    }
  };
  // Every wave stores all RT tiles unconditionally (the same number of
  // stores on every path keeps the compiler's count of memory operations in
  // flight exact, so the next item's loads stay in flight across them): a
  // spare tile past NT is a bit-identical copy of tile NT - 1 (same inputs,
  // same operations) and rewrites its bytes.
  // With `rehearse` the same stores all go to the lane's own first slot
  // (ct = 0 of its first tile, which the item's real epilogue rewrites
  // later): issued once after the prologue's loads, they give the first
  // item the same memory operations in flight as every later item, whose
  // loads were issued before the previous item's stores.  The compiler then
  // waits at one count for both, not the smaller one for both.
  auto epilogue = [&](const GramItem& it, bool rehearse) {
    // an opaque zero: the compiler cannot merge the rehearsal's stores
    int zero_s;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero_s));
    const int jm = rehearse ? zero_s : 1;
    const int h = it.h0 + hp;
    const int t = a.t0 + it.tl;
    const long pbase =
        ((((long)it.sp * a.B + it.b) * a.H + h) * a.Tc + it.tl) * NR * (long)(D * D);
    const long obase = (((long)it.b * a.H + h) * a.T + t) * (long)(D * D);
    if constexpr (SPLIT) {
#pragma unroll
      for (int j = 0; j < C::RT; ++j) {
        const int m = (j / C::RPM) * jm;
        const int ft = min(wl + C::WPH * (j % C::RPM) * jm, NT - 1);
        const float sc = (m == 0 ? a.scale0 : a.scale1);
        float* out = a.part + pbase + m * (long)(D * D) + (ft * NT * 64 + lane) * 4;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          *reinterpret_cast<f32x4*>(out + ct * 256 * jm) = sc * acc[j][ct];
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::RT; ++j) {
        const int m = (j / C::RPM) * jm;
        const int ft = min(wl + C::WPH * (j % C::RPM) * jm, NT - 1);
        const float sc = (m == 0 ? a.scale0 : a.scale1);
        E* out = static_cast<E*>(m == 0 ? a.out0 : a.out1) + obase;
        const int lay = m == 0 ? a.layout0 : a.layout1;
        // tiles: tile [ft][ct], this lane's slot; row-major or fragments
        // (transposed tile): row 16 ct + i, columns 16 ft + 4g .. + 3.  All
        // are base + ct * stride.
        E* base = lay == LAYOUT_TILES ? out + (ft * NT * 64 + lane) * 4
                  : lay == LAYOUT_FRAG ? out + frag_index(li, ft * 16 + 4 * g, D)
                                       : out + li * D + ft * 16 + 4 * g;
        const int stride = (lay == LAYOUT_TILES ? 256 : 16 * D) * jm;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) pack(sc * acc[j][ct], base + ct * stride);
      }
    }
  };

  // Persistent: this workgroup walks items v = blockIdx.x + k gridDim.x
  // (gridDim.x a multiple of 8 keeps them on this workgroup's XCD, and
  // xcd_item gives each XCD a contiguous range: neighbouring heads of one
  // frame run together).  Each item takes ncp ring steps, trips of PF (its
  // chunk count rounded up; steps past its last chunk only keep the ring in
  // step).  Step c: commit ring slot c % PF to the stage the previous real
  // step did not use (free: its last readers finished before that step's
  // barrier), barrier, reload the slot with the chunk PF steps ahead - the
  // next item's first chunks at the end of an item, so they are in flight
  // while the item's results are stored - and multiply.  The stage parity
  // runs on across items: two consecutive real steps never share a stage
  // whatever the chunk counts.
  const int G = gridDim.x;
  int v = blockIdx.x;
  if (v >= total) return;
  GramItem cur = decode(v);
  GramItem nxt = decode(v + G < total ? v + G : v);
  Ring ring[PF];
  int par = 0;
  auto trip = [&](int c0) {
#pragma unroll
    for (int r = 0; r < PF; ++r) {
      const int c = c0 + r;
      const bool real = c < cur.n;
      if (real) {
        commit(ring[r], par, N - (cur.cbeg + c) * CT);
        lds_barrier();
      }
      // PF steps ahead: this item, or the next one's first chunks
      const bool here = c + PF < ncp;
      load(ring[r], here ? cur : nxt, here ? c + PF : c + PF - ncp);
      if (real) {
        compute(par);
        par ^= 1;
      }
    }
  };
#pragma unroll
  for (int r = 0; r < PF; ++r) load(ring[r], cur, r);
  zero_acc();
  epilogue(cur, true);
  for (;;) {
    // the first trip runs after the stores on every path, the loop of the
    // other trips after the first trip's waits
    trip(0);
    for (int c0 = PF; c0 < ncp; c0 += PF) trip(c0);
    epilogue(cur, false);
    zero_acc();
    v += G;
    if (v >= total) break;
    cur = nxt;
    nxt = decode(v + G < total ? v + G : v);
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
    const bool frag = (m == 0 ? a.layout0 : a.layout1) == LAYOUT_FRAG;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int R = ft * 16 + 4 * g + r, Cc = ct * 16 + li;
      E* dst = out + (frag ? frag_index(R, Cc, D) : (long)R * D + Cc);
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

// Resident workgroups of the Gram kernel: one per CU with head pairs, two
// with single heads.
static int gram_slots(int hpw) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return cus * (hpw == 2 ? 1 : 2);
}

template <int IO, int NT, int NR, bool YX, int HPW, bool SPLIT, bool NORM>
static void launch_one(const GramArgs& a, int grid, hipStream_t s) {
  typedef GramCfg<IO, NT, NR, YX, HPW, NORM> C;
  hipLaunchKernelGGL((gram_kernel<IO, NT, NR, YX, HPW, SPLIT, NORM>), dim3(grid),
                     dim3(64 * C::WPH * HPW), 0, s, a);
}

template <int IO, int NT, int HPW>
static void launch_gram_hpw(const GramArgs& a, int nr, hipStream_t s) {
  // persistent: at most one workgroup per slot, a multiple of 8 so that a
  // workgroup's items stay on its XCD
  const int total = a.B * a.Tc * (a.H / HPW) * a.P;
  int grid = gram_slots(HPW);
  grid -= grid % 8;
  if (total < grid) grid = total;
  if (a.P > 1) {
    if (nr == 2 && a.norm)
      launch_one<IO, NT, 2, true, HPW, true, true>(a, grid, s);
    else if (nr == 2)
      launch_one<IO, NT, 2, true, HPW, true, false>(a, grid, s);
    else
      launch_one<IO, NT, 1, false, HPW, true, false>(a, grid, s);
  } else {
    if (nr == 2 && a.norm)
      launch_one<IO, NT, 2, true, HPW, false, true>(a, grid, s);
    else if (nr == 2)
      launch_one<IO, NT, 2, true, HPW, false, false>(a, grid, s);
    else
      launch_one<IO, NT, 1, false, HPW, false, false>(a, grid, s);
  }
}

template <int IO, int NT>
static hipError_t launch_gram_nt(const GramArgs& a, int nr, hipStream_t s) {
  // adjacent head pairs when H is even: each token's two row segments are
  // one contiguous, 64-byte aligned piece of memory
  if (a.H % 2 == 0)
    launch_gram_hpw<IO, NT, 2>(a, nr, s);
  else
    launch_gram_hpw<IO, NT, 1>(a, nr, s);
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
  if (a.norm && nr != 2) return hipErrorInvalidValue;
  return io == IO_BF16 ? launch_gram_io<IO_BF16>(a, nt, nr, s)
                       : launch_gram_io<IO_F32>(a, nt, nr, s);
}

}  // namespace gdn
