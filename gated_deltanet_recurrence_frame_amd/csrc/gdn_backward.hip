// Backward of the frame-wise GDN (reverse mode of the recurrence on the
// summary page, 方法步骤详情 module 2; the pages give no backward, these are
// the chain-rule gradients).  With G_t = dLoss/dS_t (from the reverse scan)
// and S_t the forward states (S_{-1} = S_0 the initial state):
//   dM_t     = S_{t-1}^T G_t            dgamma_t = tr(dM_t)
//   W_t      = dM_t + dM_t^T            (gradient of the symmetric Gram)
//   dq_n     = S_t^T do_n
//   y_n      = G_t k^_n                  dv_n = beta_n y_n
//   z_n      = G_t^T v_n                 w_n = W_t k^_n
//   dk_n     = s beta_n (z_n - w_n)
//   dbeta_n  = v_n . y_n - 1/2 k^_n . w_n   (= v^T G k^ - k^^T dM k^)
// with k^ = s k.
//
// Per-frame matrices are in the intermediate type (bf16 for bf16 io, fp32
// for fp32 io).
// dm_kernel (fp32 io): one workgroup per frame forms dM_t on MFMA from
// S_{t-1} and G_t staged in LDS, writes W_t and dgamma_t (a fixed-order
// block sum).  With bf16 io the dK/dV pass forms them itself (below).
// dQ = S_t^T dO is the output kernel run on S_t^T (gdn_output.hip).
// bwd_kv_kernel: dK, dV and dbeta by token chunks (described below).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT>
__global__ __launch_bounds__(256) void dm_kernel(DmArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr int D = 16 * NT;
  constexpr int NCT = (NT + 3) / 4;
  constexpr int KP = BF ? ((D + 31) / 32) * 32 : D;   // contraction rows, zero padded
  constexpr int LD = D + 1;                           // padded fp32 row for dM
  constexpr int IN_BYTES = 2 * KP * (BF ? D : LD) * (BF ? 2 : 4);
  constexpr int DM_BYTES = D * LD * 4;
  constexpr int SMEM = IN_BYTES > DM_BYTES ? IN_BYTES : DM_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ float red[256];

  const int total = a.B * a.T * a.H;
  const int item = xcd_item(blockIdx.x, total);
  const int h = item % a.H;
  const int t = (item / a.H) % a.T;
  const int b = item / (a.H * a.T);
  const long DD = (long)D * D;
  const long bh = (long)b * a.H + h;
  const E* Sp = t > 0 ? static_cast<const E*>(a.S) + (bh * a.T + t - 1) * DD : nullptr;
  const float* S0 = (t == 0 && a.s0) ? a.s0 + bh * DD : nullptr;
  const E* Gt = static_cast<const E*>(a.G) + (bh * a.T + t) * DD;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int g = lane >> 4, li = lane & 15;

  // Stage S_{t-1} and G_t (intermediate type; S_0 rounded like the saved
  // states) and accumulate dgamma_t = <S_{t-1}, G_t>.
  E* Sl = reinterpret_cast<E*>(smem);
  E* Gl = Sl + KP * (BF ? D : LD);
  const int SLD = BF ? D : LD;
  float dot = 0.f;
  if constexpr (BF) {
    // 8 values (16 bytes) per step; rows past D are zero.
    constexpr int PRW = D / 8;
    for (int p = tid; p < KP * PRW; p += 256) {
      const int i = p / PRW, j = (p % PRW) * 8;
      u32x4 gv = {0u, 0u, 0u, 0u}, sv = {0u, 0u, 0u, 0u};
      if (i < D) {
        gv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(Gt) + i * D + j);
        if (Sp) {
          sv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(Sp) + i * D + j);
        } else if (S0) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(S0 + i * D + j);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(S0 + i * D + j + 4);
          float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          sv = __builtin_bit_cast(u32x4, f32x8_to_bf16x8(v));
        }
      }
      const bf16x8 gb = __builtin_bit_cast(bf16x8, gv), sb = __builtin_bit_cast(bf16x8, sv);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += static_cast<float>(sb[e]) * static_cast<float>(gb[e]);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(Sl) + i * SLD + j) = sv;
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(Gl) + i * SLD + j) = gv;
    }
  } else {
    for (int idx = tid; idx < D * D; idx += 256) {
      const int i = idx / D, j = idx % D;
      const float gv = reinterpret_cast<const float*>(Gt)[idx];
      const float sv = Sp ? reinterpret_cast<const float*>(Sp)[idx] : (S0 ? S0[idx] : 0.f);
      reinterpret_cast<float*>(Sl)[i * SLD + j] = sv;
      reinterpret_cast<float*>(Gl)[i * SLD + j] = gv;
      dot += sv * gv;
    }
  }
  red[tid] = dot;
  block_sync();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    block_sync();
  }
  if (tid == 0) a.dgamma[((long)b * a.T + t) * a.H + h] = red[0];

  // dM[j][l] = sum_i S[i][j] G[i][l]; this wave's row tiles jt = wave + 4j.
  f32x4 acc[NCT][NT];
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int lt = 0; lt < NT; ++lt) acc[j][lt] = zero4();
  if constexpr (BF) {
    const uint16_t* S16 = reinterpret_cast<const uint16_t*>(Sl);
    const uint16_t* G16 = reinterpret_cast<const uint16_t*>(Gl);
#pragma unroll
    for (int kb = 0; kb < KP / 32; ++kb) {
      bf16x8 gb[NT];
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) gb[lt] = lds_col_frag_bf16(G16, D, kb * 32, lt * 16);
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const int jt = wave + 4 * j;
        if (jt < NT) {
          const bf16x8 af = lds_col_frag_bf16(S16, D, kb * 32, jt * 16);
#pragma unroll
          for (int lt = 0; lt < NT; ++lt) acc[j][lt] = mfma_bf16(af, gb[lt], acc[j][lt]);
        }
      }
    }
  } else {
    const float* Sf = reinterpret_cast<const float*>(Sl);
    const float* Gf = reinterpret_cast<const float*>(Gl);
#pragma unroll 2
    for (int kb = 0; kb < D / 4; ++kb) {
      const int i = kb * 4 + g;
      float gb[NT];
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) gb[lt] = Gf[i * LD + lt * 16 + li];
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const int jt = wave + 4 * j;
        if (jt < NT) {
          const float av = Sf[i * LD + jt * 16 + li];
#pragma unroll
          for (int lt = 0; lt < NT; ++lt) acc[j][lt] = mfma_f32(av, gb[lt], acc[j][lt]);
        }
      }
    }
  }
  block_sync();
  // Stage dM (padded fp32 rows) and emit W = dM + dM^T.
  float* dm = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int jt = wave + 4 * j;
    if (jt < NT) {
#pragma unroll
      for (int lt = 0; lt < NT; ++lt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dm[(jt * 16 + 4 * g + r) * LD + lt * 16 + li] = acc[j][lt][r];
    }
  }
  block_sync();
  E* Wt = static_cast<E*>(a.W) + (bh * a.T + t) * DD;
  // 8 consecutive entries of a row of W per step, one 16-byte (bf16) or two
  // 16-byte (fp32) stores.
  for (int p = tid; p < D * D / 8; p += 256) {
    const int j = p / (D / 8), l = (p % (D / 8)) * 8;
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = dm[j * LD + l + e] + dm[(l + e) * LD + j];
    if constexpr (BF) {
      *reinterpret_cast<bf16x8*>(reinterpret_cast<uint16_t*>(Wt) + j * D + l) = f32x8_to_bf16x8(w);
    } else {
      float* dst = reinterpret_cast<float*>(Wt) + j * D + l;
      *reinterpret_cast<f32x4*>(dst) = f32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{w[4], w[5], w[6], w[7]};
    }
  }
}

// bwd_kv_kernel: one workgroup per (b, t) frame and group of HPW adjacent
// heads (pairs when H is even: a token's two head rows are one contiguous
// 448-byte piece at D = 112, where single-head rows half-fill their first
// or last 64-byte sector), one wave per (head, 16-feature tile).  Each wave
// keeps its rows of G_t, G_t^T and W_t as MFMA operands in registers.
// Token rows of K and V stream in chunks of CT tokens: each thread loads
// its 16-byte pieces of a chunk into a register ring PF chunks deep,
// commits them to a double-buffered LDS stage behind an LDS-only barrier
// (the ring stays in flight across it), and every wave reads its head's
// rows of the chunk as the other MFMA operand.  dK and dV are staged in
// LDS and stored one chunk later as contiguous 16-byte pieces of token
// rows; dbeta sums the per-feature-tile partial dot products in a fixed
// order (deterministic, no atomics).
// With normalised keys (CHAIN, bf16) the pass reads the raw key rows: the
// thread that commits a 16-byte piece of a key row to LDS also stages the sum
// of its eight squares, and every wave adds its tokens' piece sums in a fixed
// order, so it has |k| per token without a K K^T product of its own; its
// products with k (per-token columns) and k itself are scaled by
// iv = 1 / |k| (0 for a zero row).  The normalisation's chain rule,
//   dk = (dk^ - k^ (k^ . dk^)) iv = g - k (iv (k^ . g)),  g = iv dk^,
// takes g from the compute step (iv folds into its per-token factor), staged
// in bf16 like dV, and k^ . g summed over the feature tiles in a fixed order;
// the store then spends one FMA per element.
// Registers bound the shape: at 14 waves per CU a wave has 128 VGPRs, of
// which its three matrices take 48; chunks of 16 tokens (pairs) two deep
// fit without spills (at D = 112 the whole backward went from 1.17 to
// 0.99 ms against the single-head kernel with a ring of direct-to-LDS
// copies; 32-token chunks or a third chunk in flight spilled and ran
// slower).
template <int IO, int NT, int HPW, bool CHAIN>
__global__ __launch_bounds__(64 * NT * HPW, 1) void bwd_kv_kernel(BwdTokArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int RW = HPW * D;                    // elements of a token's row segment
  constexpr int CT = BF ? 32 / HPW : 16;         // tokens per chunk (whole 16-token tiles)
  constexpr int PR = RW * ES / 16;               // 16-byte pieces per row segment
  constexpr int LDR = RW + (BF ? 8 : 4);         // padded LDS row (elements)
  constexpr int NTH = 64 * NT * HPW;
  constexpr int PPT = 2 * CT * PR / NTH;         // K and V pieces per thread per chunk
  constexpr int PF = 2;                          // chunks in flight
  constexpr int KB = BF ? (D + 31) / 32 : D / 4;
  constexpr int NB = CT * HPW;                   // gates per chunk
  static_assert(PPT * NTH == 2 * CT * PR, "pieces must split evenly over the threads");
  static_assert(CT % 16 == 0, "chunks of whole 16-token tiles");
  static_assert(NB <= NTH, "one gate per thread at most");
  // stage: K rows then V rows of a chunk (16 elements of padding: the zeroed
  // tail of a last 32-column block stays inside the array)
  constexpr int STAGE = 2 * CT * LDR + 16;
  constexpr int OBUF = 2 * CT * LDR;             // dK rows, dV rows
  constexpr int KR = KB * (BF ? 32 : 4);         // staged rows of a D x D matrix (zero past D)
  constexpr int WLD = D + 8;                     // a wave's staged W rows
  // bf16 prologue: the heads' G_t and S_{t-1} as [KR][D] rows, then every
  // wave's 16 rows of W_t
  constexpr int PRO = BF ? 2 * HPW * KR * D : HPW * KR * D;
  static_assert(!BF || NT * HPW * 16 * WLD <= PRO, "W rows fit the prologue region");
  constexpr int MAIN = 2 * STAGE + 2 * OBUF;
  // the stages and the output staging, one array, shared with the prologue
  __shared__ __attribute__((aligned(16))) E lds[MAIN > PRO ? MAIN : PRO];
  __shared__ float gred[BF ? HPW : 1][NT * HPW];   // dgamma partials per wave
  auto stage = [&](int i) { return lds + i * STAGE; };
  auto obuf = [&](int i) { return lds + 2 * STAGE + i * OBUF; };
  __shared__ float bstage[2][NB];
  __shared__ float red[2][HPW][NT][CT];                               // dbeta partials
  static_assert(!CHAIN || BF, "the fused chain rule is for bf16");
  // k^ . g partials per token, the tiles' side by side (two 16-byte reads)
  __shared__ __attribute__((aligned(16))) float cred[CHAIN ? 2 : 1][HPW][CT][8];
  static_assert(NT <= 8, "the partials' row holds eight tiles");
  __shared__ float istage[CHAIN ? 2 : 1][NB];                         // 1 / |k| per token, head
  constexpr int KP = D / 8;                                            // key pieces per head row
  __shared__ float ksq[CHAIN ? 2 : 1][CHAIN ? CT * PR : 1];            // squares per key piece

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
  const int hp = wave / NT, ft = wave % NT;      // this wave's head (in the group), tile
  const int g = lane >> 4, li = lane & 15;
  const float s = a.s;
  const int h = h0 + hp;
  const long moff = (((long)b * a.H + h) * a.T + t) * DD;

  // Left operands of this wave's feature tile: rows of G_t, of G_t^T
  // (columns of G_t: bf16 from G_t staged in LDS with the transposing read)
  // and of W_t (symmetric).
  const E* Gt = static_cast<const E*>(a.G) + moff;
  const int fr = ft * 16 + li;
  typedef typename std::conditional<BF, bf16x8, float>::type Frag;
  Frag mG[KB], mGT[KB], mW[KB];
  if constexpr (BF) {
    // The group's G_t and S_{t-1} (S_0 rounded like the saved states, or
    // zero) as [KR][D] rows, rows past D zero, summing dgamma_t = <S_{t-1},
    // G_t> on the way; then every wave forms its 16 rows of
    //   W_t = S_{t-1}^T G_t + G_t^T S_{t-1}  (= dM_t + dM_t^T)
    // on MFMA (columns of both staged matrices by the transposing read; the
    // second product's left operand is the G_t^T fragments the wave keeps),
    // stages them in LDS and reads them back as operand rows.
    uint16_t* Gs = reinterpret_cast<uint16_t*>(lds);
    uint16_t* Ss = Gs + HPW * KR * D;
    constexpr int PRW = D / 8;
    float dot[HPW];
#pragma unroll
    for (int m = 0; m < HPW; ++m) dot[m] = 0.f;
    for (int p = tid; p < HPW * KR * PRW; p += NTH) {
      const int m = p / (KR * PRW), r = p % (KR * PRW);
      const int row = r / PRW, pc = r % PRW;
      const long bhm = (long)b * a.H + h0 + m;
      u32x4 gv = {0u, 0u, 0u, 0u}, sv = {0u, 0u, 0u, 0u};
      if (row < D) {
        gv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.G) + (bhm * a.T + t) * DD +
                                             row * D + pc * 8);
        if (t > 0) {
          sv = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.S) +
                                               (bhm * a.T + t - 1) * DD + row * D + pc * 8);
        } else if (a.s0) {
          const float* s0 = a.s0 + bhm * DD + row * D + pc * 8;
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(s0);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(s0 + 4);
          float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          sv = __builtin_bit_cast(u32x4, f32x8_to_bf16x8(x));
        }
      }
      const bf16x8 gb = __builtin_bit_cast(bf16x8, gv), sb = __builtin_bit_cast(bf16x8, sv);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += static_cast<float>(sb[e]) * static_cast<float>(gb[e]);
#pragma unroll
      for (int mm = 0; mm < HPW; ++mm) dot[mm] += mm == m ? d : 0.f;
      *reinterpret_cast<u32x4*>(Gs + (m * KR + row) * D + pc * 8) = gv;
      *reinterpret_cast<u32x4*>(Ss + (m * KR + row) * D + pc * 8) = sv;
    }
    // dgamma partials: a fixed-order sum within each wave, then over the waves
#pragma unroll
    for (int m = 0; m < HPW; ++m) {
      float v = dot[m];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) gred[m][wave] = v;
    }
    block_sync();
    const uint16_t* Gh = Gs + hp * KR * D;
    const uint16_t* Sh = Ss + hp * KR * D;
    f32x4 wacc[NT];
    {
      bf16x8 sT[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k = kb * 32 + 8 * g;
        mGT[kb] = lds_col_frag_bf16(Gh, D, kb * 32, ft * 16);
        sT[kb] = lds_col_frag_bf16(Sh, D, kb * 32, ft * 16);
        mG[kb] = (k < D) ? load_bf16x8(Gh + fr * D + k) : zero_bf16x8();
      }
#pragma unroll
      for (int lt = 0; lt < NT; ++lt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          acc = mfma_bf16(sT[kb], lds_col_frag_bf16(Gh, D, kb * 32, lt * 16), acc);
          acc = mfma_bf16(mGT[kb], lds_col_frag_bf16(Sh, D, kb * 32, lt * 16), acc);
        }
        wacc[lt] = acc;
      }
    }
    if (tid < HPW) {
      float sum = 0.f;
      for (int w = 0; w < NT * HPW; ++w) sum += gred[tid][w];
      a.dgamma[((long)b * a.T + t) * a.H + h0 + tid] = sum;
    }
    block_sync();   // every wave is done with the staged G_t, S_{t-1}
    uint16_t* Wr = reinterpret_cast<uint16_t*>(lds) + wave * 16 * WLD;
#pragma unroll
    for (int lt = 0; lt < NT; ++lt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Wr[(4 * g + r) * WLD + lt * 16 + li] = f32_to_bf16_bits(wacc[lt][r]);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 32 + 8 * g;
      mW[kb] = (k < D) ? load_bf16x8(Wr + li * WLD + k) : zero_bf16x8();
    }
    block_sync();   // the LDS is the chunk loop's from here on
  } else {
    const E* Wt = static_cast<const E*>(a.W) + moff;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 4 + g;
      mG[kb] = Gt[fr * D + k];
      mGT[kb] = Gt[k * D + fr];
      mW[kb] = Wt[fr * D + k];
    }
  }

  const int nchunks = (N + CT - 1) / CT;
  // Addresses: a uniform 64-bit base of the frame's rows of the head group
  // plus 32-bit per-lane offsets from 24-bit multiplies (the host keeps a
  // frame's rows under 2 GiB and N, H D es under 2^24).
  const long fbase = (row0 * a.H + h0) * (long)(D * ES);
  const char* kframe = static_cast<const char*>(a.k) + fbase;
  const char* vframe = static_cast<const char*>(a.v) + fbase;
  char* dkframe = static_cast<char*>(a.dk) + fbase;
  char* dvframe = static_cast<char*>(a.dv) + fbase;
  const float* bframe = a.beta + row0 * a.H + h0;
  float* dbframe = a.dbeta + row0 * a.H + h0;
  const unsigned rowb = (unsigned)(a.H * D * ES);   // bytes between tokens
  struct Ring {
    u32x4 v[PPT];
    float bt;
  };
  // Chunk c: piece p = tid + NTH j of [K rows | V rows] (row p / PR of
  // matrix (p / (CT PR))), rows past the frame re-read its last row.
  auto issue = [&](Ring& R, int c) {
    const int c0 = (c < nchunks ? c : nchunks - 1) * CT;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      const int m = p / (CT * PR), r = p % (CT * PR);
      const int row = r / PR, pc = r % PR;
      int tk = c0 + row;
      if (tk >= N) tk = N - 1;
      const unsigned off = __umul24((unsigned)tk, rowb) + (unsigned)(pc * 16);
      R.v[j] = *reinterpret_cast<const u32x4*>((m ? vframe : kframe) + off);
    }
    const int bi = tid < NB ? tid : 0;
    int tk = c0 + bi / HPW;
    if (tk >= N) tk = N - 1;
    R.bt = bframe[__umul24((unsigned)tk, (unsigned)a.H) + (unsigned)(bi % HPW)];
  };
  auto commit = [&](const Ring& R, int c) {
    E* st = stage(c & 1);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      const int m = p / (CT * PR), r = p % (CT * PR);
      *reinterpret_cast<u32x4*>(st + (m * CT + r / PR) * LDR + (r % PR) * (16 / ES)) = R.v[j];
      if constexpr (CHAIN) {
        if (m == 0) {
          float q = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = __uint_as_float(R.v[j][e] << 16);
            const float x1 = __uint_as_float(R.v[j][e] & 0xffff0000u);
            q += x0 * x0 + x1 * x1;
          }
          ksq[c & 1][r] = q;
        }
      }
    }
    // tokens past the frame's end get gate 0 (their rows are re-read copies)
    if (tid < NB) bstage[c & 1][tid] = c * CT + tid / HPW < N ? R.bt : 0.f;
  };
  auto load4 = [&](const E* row) -> f32x4 {   // 4 values at this lane's features
    f32x4 r;
    if constexpr (BF) {
      const u32x2 pk = *reinterpret_cast<const u32x2*>(row + ft * 16 + 4 * g);
      r[0] = bf16_bits_to_f32((uint16_t)(pk[0] & 0xffff));
      r[1] = bf16_bits_to_f32((uint16_t)(pk[0] >> 16));
      r[2] = bf16_bits_to_f32((uint16_t)(pk[1] & 0xffff));
      r[3] = bf16_bits_to_f32((uint16_t)(pk[1] >> 16));
    } else {
      r = *reinterpret_cast<const f32x4*>(row + ft * 16 + 4 * g);
    }
    return r;
  };
  auto put4 = [&](E* dst, const f32x4& v) {
    if constexpr (BF) {
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
      *reinterpret_cast<f32x4*>(dst) = v;
    }
  };
  auto compute = [&](int c) {
    const E* ks = stage(c & 1) + hp * D;
    const E* vs = stage(c & 1) + CT * LDR + hp * D;
    const float* bs = bstage[c & 1];
    E* ob = obuf(c & 1);
    // one 16-token tile at a time (hoisting every tile's fragments would
    // not fit the registers of 14 waves per CU)
#pragma unroll 1
    for (int tt = 0; tt < CT / 16; ++tt) {
      const int trow = tt * 16 + li;
      f32x4 ay = zero4(), az = zero4(), aw = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (BF) {
          const int k = kb * 32 + 8 * g;
          // past D the read runs into the next head or the padding: zero it
          const bool ok = k < D;
          const bf16x8 kf = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(ks + trow * LDR) + k)
                               : zero_bf16x8();
          const bf16x8 vf = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(vs + trow * LDR) + k)
                               : zero_bf16x8();
          ay = mfma_bf16(mG[kb], kf, ay);
          az = mfma_bf16(mGT[kb], vf, az);
          aw = mfma_bf16(mW[kb], kf, aw);
          // one block's fragments live at a time (registers)
          __builtin_amdgcn_sched_barrier(0);
        } else {
          const int k = kb * 4 + g;
          const float kf = ks[trow * LDR + k];
          const float vf = vs[trow * LDR + k];
          ay = mfma_f32(mG[kb], kf, ay);
          az = mfma_f32(mGT[kb], vf, az);
          aw = mfma_f32(mW[kb], kf, aw);
        }
      }
      const float bt = bs[trow * HPW + hp];
      float iv = 1.f;   // CHAIN: 1 / |k| of token trow (the staged k row is raw)
      const f32x4 kv = load4(ks + trow * LDR);
      const f32x4 vv = load4(vs + trow * LDR);
      if constexpr (CHAIN) {
        // |k|^2 of token trow: lane group g adds pieces g, g + 4, ... of the
        // head's row, then the four groups' sums (the same order in every lane)
        const float* kq = ksq[c & 1] + trow * PR + hp * KP;
        float sq = 0.f;
#pragma unroll
        for (int q = 0; q < (KP + 3) / 4; ++q)
          if (g + 4 * q < KP) sq += kq[g + 4 * q];
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        iv = inv_norm(sq);
        if (ft == 0 && g == 0) istage[c & 1][trow * HPW + hp] = iv;
      }
      // per-token factors: ay, aw and k carry iv under CHAIN (k^ = iv k), and
      // dK^ = s bt (az - w) is formed as g = iv dK^ there
      const float sy = s * iv, hk = 0.5f * s * iv, sk = s * bt * iv;
      f32x4 dvv, dkv;
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = sy * ay[r];         // (G k^)_f
        const float w = sy * aw[r];         // (W k^)_f
        dvv[r] = bt * y;
        dkv[r] = sk * (az[r] - w);
        part += vv[r] * y - hk * kv[r] * w;
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (g == 0) red[c & 1][hp][ft][trow] = part;
      if constexpr (CHAIN) {
        float cp = iv * (kv[0] * dkv[0] + kv[1] * dkv[1] + kv[2] * dkv[2] + kv[3] * dkv[3]);
        cp += __shfl_xor(cp, 16);
        cp += __shfl_xor(cp, 32);
        if (g == 0) cred[c & 1][hp][trow][ft] = cp;
      }
      put4(ob + trow * LDR + hp * D + ft * 16 + 4 * g, dkv);
      put4(ob + CT * LDR + trow * LDR + hp * D + ft * 16 + 4 * g, dvv);
    }
  };
  // dK, dV pieces and dbeta of chunk c (staged by compute(c))
  auto store = [&](int c, bool full) {
    const E* src = obuf(c & 1);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      const int m = p / (CT * PR), r = p % (CT * PR);
      const int row = r / PR, pc = r % PR;
      const int tk = c * CT + row;
      const unsigned off = __umul24((unsigned)tk, rowb) + (unsigned)(pc * 16);
      u32x4 v = *reinterpret_cast<const u32x4*>(src + (m * CT + row) * LDR + pc * (16 / ES));
      if constexpr (CHAIN) {
        if (m == 0) {
          // dk = g - k (iv (k^ . g)) on this piece of head hm's row (k raw)
          const int hm = pc / (D / 8);
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(&cred[c & 1][hm][row][0]);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(&cred[c & 1][hm][row][4]);
          const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
          float dot = 0.f;
#pragma unroll
          for (int f = 0; f < NT; ++f) dot += cv[f];
          const float cf = istage[c & 1][row * HPW + hm] * dot;
          const u32x4 kx = *reinterpret_cast<const u32x4*>(stage(c & 1) + row * LDR + pc * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g0 = __uint_as_float(v[e] << 16), g1 = __uint_as_float(v[e] & 0xffff0000u);
            const float k0 = __uint_as_float(kx[e] << 16);
            const float k1 = __uint_as_float(kx[e] & 0xffff0000u);
            const f32x2 d = {g0 - k0 * cf, g1 - k1 * cf};
            v[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(d, bf16x2));
          }
        }
      }
      if (full || tk < N) *reinterpret_cast<u32x4*>((m ? dvframe : dkframe) + off) = v;
    }
    if (tid < NB) {
      const int tk = c * CT + tid / HPW, m = tid % HPW;
      float sum = 0.f;
#pragma unroll
      for (int f = 0; f < NT; ++f) sum += red[c & 1][m][f][tid / HPW];
      if (full || tk < N) dbframe[__umul24((unsigned)tk, (unsigned)a.H) + (unsigned)m] = sum;
    }
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
}

template <int IO, int NT>
static hipError_t launch_dm_nt(const DmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((dm_kernel<IO, NT>), dim3(a.B * a.T * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_dm_io(const DmArgs& a, int nt, hipStream_t s) {
  switch (nt) {
    case 1: return launch_dm_nt<IO, 1>(a, s);
    case 2: return launch_dm_nt<IO, 2>(a, s);
    case 3: return launch_dm_nt<IO, 3>(a, s);
    case 4: return launch_dm_nt<IO, 4>(a, s);
    case 5: return launch_dm_nt<IO, 5>(a, s);
    case 6: return launch_dm_nt<IO, 6>(a, s);
    case 7: return launch_dm_nt<IO, 7>(a, s);
    case 8: return launch_dm_nt<IO, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dm(const DmArgs& a, int io, int nt, hipStream_t s) {
  return io == IO_BF16 ? launch_dm_io<IO_BF16>(a, nt, s) : launch_dm_io<IO_F32>(a, nt, s);
}

template <int IO, int NT, bool CHAIN>
static void launch_bwd_tok_chain(const BwdTokArgs& a, hipStream_t s) {
  // adjacent head pairs when H is even (bf16: fp32's three D x D operand
  // matrices would not fit the registers of 14 waves per CU)
  if (IO == IO_BF16 && a.H % 2 == 0)
    hipLaunchKernelGGL((bwd_kv_kernel<IO, NT, 2, CHAIN>), dim3(a.B * a.T * (a.H / 2)),
                       dim3(128 * NT), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<IO, NT, 1, CHAIN>), dim3(a.B * a.T * a.H), dim3(64 * NT), 0,
                       s, a);
}
template <int IO, int NT>
static hipError_t launch_bwd_tok_nt(const BwdTokArgs& a, hipStream_t s) {
  if constexpr (IO == IO_BF16) {
    if (a.norm) {
      launch_bwd_tok_chain<IO, NT, true>(a, s);
      return hipGetLastError();
    }
  } else {
    if (a.norm) return hipErrorInvalidValue;   // normalised raw keys: bf16 only
  }
  launch_bwd_tok_chain<IO, NT, false>(a, s);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_bwd_tok_io(const BwdTokArgs& a, int nt, hipStream_t s) {
  switch (nt) {
    case 1: return launch_bwd_tok_nt<IO, 1>(a, s);
    case 2: return launch_bwd_tok_nt<IO, 2>(a, s);
    case 3: return launch_bwd_tok_nt<IO, 3>(a, s);
    case 4: return launch_bwd_tok_nt<IO, 4>(a, s);
    case 5: return launch_bwd_tok_nt<IO, 5>(a, s);
    case 6: return launch_bwd_tok_nt<IO, 6>(a, s);
    case 7: return launch_bwd_tok_nt<IO, 7>(a, s);
    case 8: return launch_bwd_tok_nt<IO, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tok(const BwdTokArgs& a, int io, int nt, hipStream_t s) {
  return io == IO_BF16 ? launch_bwd_tok_io<IO_BF16>(a, nt, s)
                       : launch_bwd_tok_io<IO_F32>(a, nt, s);
}

}  // namespace gdn
