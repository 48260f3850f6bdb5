// Token-space form of the frame-wise GDN forward, for frames with few tokens.
//
// Same recurrence as the frame form (summary page: 前置知识 "Gated DeltaNet"
// and 方法步骤详情 module 2), S_t = S_{t-1}(gamma_t I - K^_t beta_t K^_t^T)
// + V_t beta_t K^_t^T, O_t = S_t Q^_t, evaluated over chunks of F frames
// (C = F N <= CP tokens) without any D x D product per frame.  Per chunk,
// with E_0 the entering state, f(t) the frame of token t in the chunk and
// P(a, b) = gamma_a ... gamma_b (1 when a > b):
//   w_t = (v_t - E_{f(t)} k^_t) beta_t         corrected values, W (I + L) = R:
//   R[:, t] = (v_t - P(0, f(t)-1) E_0 k^_t) beta_t
//   L[u, t] = P(f(u)+1, f(t)-1) (k^_u . k^_t) beta_t  for f(u) < f(t), else 0
//   o_t     = P(0, f(t)) E_0 q_t + sum_{f(u) <= f(t)} P(f(u)+1, f(t)) w_u (k^_u . q_t)
//   E_F     = P(0, F-1) E_0 + sum_u P(f(u)+1, F-1) w_u k^_u^T.
// L is strictly upper triangular in token order (a frame's tokens do not see
// each other), so I + L is unit upper triangular.
//
// Two kernels.  Everything that depends only on a chunk's own K, Q, beta
// and gamma - the inverse (I + L)^-1 (substitution on 16 x 16 diagonal
// blocks, block back-substitution above them, fp32), the output mixing
// Om[u, t] = P(f(u)+1, f(t)) (k^_u . q_t) and the per-token decays - is
// computed for all chunks at once (token_prep_kernel, one workgroup per
// (b, h, chunk)) into the workspace.  The state pass (token_scan_kernel,
// one workgroup per (b, h), one wave per 16 state rows) then only does
// what depends on the state, chunk after chunk:
//   SK = E_0 K^T, SQ = E_0 Q^T, R, W = R (I + L)^-1, O = P(0, f) SQ + W Om,
//   E_F = P(0, F-1) E_0 + s (W tail) K,
// with the next chunk's inputs in flight in a register ring.  Long
// sequences are cut into segments of chunks walked in parallel: a composite
// pass per segment (the input composite H from a zero state, the transition
// composite Phi from the identity without inputs - [RB] 技术新颖性 point 1's
// context-parallel composites, with segments in place of devices), the
// frame form's fold of the composites, and a replay of every segment from
// its entering state.
// bf16 io: bf16 MFMA 16x16x32 with fp32 accumulation, the state and W
// rounded to bf16 as MFMA operands (as in the frame form's scan); fp32 io:
// fp32 MFMA 16x16x4 throughout.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT>
struct TokLayout {
  typedef typename Io<IO>::elem E;
  static constexpr bool BF = (IO == IO_BF16);
  static constexpr int D = 16 * NT;
  static constexpr int CP = TokCfg<IO>::CP;
  static constexpr int NB = CP / 16;
  static constexpr int KS = BF ? 32 : 4;              // MFMA contraction depth
  static constexpr int DP = (D + KS - 1) / KS * KS;   // feature dim padded to KS (zeros)
  static constexpr int PAD = BF ? 8 : 4;              // 16 bytes
  static constexpr int KLD = DP + PAD;                // K, Q rows in LDS
  static constexpr int FLD = CP + 1;                  // fp32 token x token matrices
  static constexpr int TLD = CP + PAD;                // MFMA copies of them
  static constexpr int ES = Io<IO>::bytes;
  static constexpr int PR = D * ES / 16;              // 16-byte pieces of a token row
  static constexpr int EP = 16 / ES;                  // elements per piece
  static constexpr int CPR = CP * ES / 16;            // pieces of a CP-element row
};

// ---------------------------------------------------------------------------
// Per-chunk operators, one workgroup of 8 waves per (b, h, chunk).  Record
// (b, h, chunk) of the workspace: TiT[t][u] = (I + L)^-1[u][t], OmT[t][u] =
// Om[u][t] (CP x CP each, io type), then 5 x CP floats: P(0, f(t) - 1),
// P(0, f(t)), P(f(t) + 1, F - 1), beta_t, and P(0, F - 1) first in the last.
template <int IO, int NT>
__global__ __launch_bounds__(512) void token_prep_kernel(TokArgs a) {
  typedef TokLayout<IO, NT> Y;
  typedef typename Y::E E;
  constexpr bool BF = Y::BF;
  constexpr int D = Y::D, CP = Y::CP, NB = Y::NB, KS = Y::KS, DP = Y::DP;
  constexpr int FLD = Y::FLD;
  constexpr int NW = 8, NTH = 512;

  constexpr int KLD = Y::KLD, EP = Y::EP;
  constexpr int PRD = D * Y::ES / 16;                 // 16-byte pieces of a row inside D
  constexpr int PRP = DP * Y::ES / 16;                // ... of a staged (zero-padded) row
  constexpr int NPC = 2 * CP * PRP;                   // staged pieces of K and Q
  constexpr int NPJ = (NPC + NTH - 1) / NTH;
  constexpr int STG = 2 * CP * KLD * Y::ES;           // K, Q rows staged
  constexpr int GRM = 2 * CP * FLD * 4;               // the two token x token matrices
  // The chunk's K and Q rows, staged; once the Gram tiles are in registers
  // the same bytes hold K^ K^^T (then L in place) and K Q^T (then (I + L)^-1).
  __shared__ __attribute__((aligned(16))) char Rg[STG > GRM ? STG : GRM];
  E* Ks = reinterpret_cast<E*>(Rg);
  E* Qs = Ks + CP * KLD;
  float* KKs = reinterpret_cast<float*>(Rg);
  float* KQs = KKs + CP * FLD;
  // Dt(x, c) = P(x, c - 1) for x <= c <= CP, rows packed (the upper
  // triangle only: three workgroups per CU fit in LDS)
  __shared__ float Dt[(CP + 1) * (CP + 2) / 2];
  __shared__ float Ys[NB][256];
  __shared__ float gs[CP], bs[CP];
  __shared__ int fr[CP];

  const int total = a.B * a.H * a.nck;
  const int item = xcd_item(blockIdx.x, total);
  const int ck = item % a.nck, bh = item / a.nck;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, T = a.T;
  const long L = (long)T * N;
  const int t0 = ck * a.F;
  const int nf = min(a.F, T - t0);
  const int C = nf * N;
  const long tok0 = (long)t0 * N;
  const float s = a.s, s2 = a.s * a.s;
  const E* K = static_cast<const E*>(a.k);
  const E* Q = static_cast<const E*>(a.q);

  auto toE = [](float x) -> E {
    if constexpr (BF) return f32_to_bf16_bits(x); else return x;
  };
  auto fragA = [&](const E* M, int ld, int m0, int k0) {
    if constexpr (BF) return load_bf16x8(M + (m0 + li) * ld + k0 + 8 * g);
    else return M[(m0 + li) * ld + k0 + g];
  };
  auto mma = [&](auto x, auto y, f32x4 c) {
    if constexpr (BF) return mfma_bf16(x, y, c); else return mfma_f32(x, y, c);
  };
  auto fence = []() {   // a wave's LDS writes land before its lanes read them back
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
  };
  // index of Dt(x, c); c < x (a value the caller discards) reads Dt(x, x)
  auto dti = [](int x, int c) { return x * (CP + 1) - x * (x - 1) / 2 + (c > x ? c - x : 0); };

  // 1. the chunk's gates and its K and Q rows (zero past C and D), every
  // load in flight at once: unconditional loads from clamped addresses, the
  // values past the chunk or the row replaced by zeros afterwards
  if (tid < CP) {
    gs[tid] = tid < nf ? a.gamma[((long)b * T + t0 + tid) * a.H + h] : 0.f;
    bs[tid] = tid < C ? a.beta[((long)b * L + tok0 + tid) * a.H + h] : 0.f;
    fr[tid] = tid / N;
  }
  {
    u32x4 pcs[NPJ];
#pragma unroll
    for (int j = 0; j < NPJ; ++j) {
      const int p = min(tid + NTH * j, NPC - 1);
      const int m = p / (CP * PRP), r = (p / PRP) % CP, pc = p % PRP;
      const long off = (((long)b * L + tok0 + min(r, C - 1)) * a.H + h) * D + min(pc, PRD - 1) * EP;
      pcs[j] = *reinterpret_cast<const u32x4*>((m ? Q : K) + off);
    }
#pragma unroll
    for (int j = 0; j < NPJ; ++j) {
      const int p = tid + NTH * j;
      if (p < NPC) {
        const int m = p / (CP * PRP), r = (p / PRP) % CP, pc = p % PRP;
        const bool in = r < C && pc < PRD;
        *reinterpret_cast<u32x4*>((m ? Qs : Ks) + r * KLD + pc * EP) =
            in ? pcs[j] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  block_sync();

  // 2. decay table: thread x runs the product over the chunk's gates, all
  // of them first read into registers; K^ K^^T on blocks i <= j and K Q^T
  // from the staged rows, into registers, then over the staged rows
  for (int x = tid; x <= nf; x += NTH) {
    float gv[CP];
#pragma unroll
    for (int c = 0; c < CP; ++c) gv[c] = gs[c];
    float p = 1.f;
    Dt[dti(x, x)] = 1.f;
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      const bool in = c >= x && c < nf;
      p = in ? p * gv[c] : p;
      if (in) Dt[dti(x, c + 1)] = p;
    }
  }
  {
    constexpr int NP = NB * (NB + 1) / 2;
    constexpr int TRIPS = (NP + NB * NB + NW - 1) / NW;
    f32x4 acc[TRIPS];
    int tile[TRIPS];
#pragma unroll
    for (int it = 0; it < TRIPS; ++it) {
      const int q = w + NW * it;
      acc[it] = zero4();
      tile[it] = -1;
      if (q < NP + NB * NB) {
        int i, j;
        const bool kq = q >= NP;
        if (kq) {
          i = (q - NP) / NB; j = (q - NP) % NB;
        } else {
          int rem = q; i = 0;
          while (rem >= NB - i) { rem -= NB - i; ++i; }
          j = i + rem;
        }
        const E* Bm = kq ? Qs : Ks;
#pragma unroll
        for (int kb = 0; kb < DP / KS; ++kb)
          acc[it] = mma(fragA(Ks, KLD, 16 * i, kb * KS), fragA(Bm, KLD, 16 * j, kb * KS), acc[it]);
        tile[it] = (kq ? 1 << 16 : 0) | (i << 8) | j;
      }
    }
    block_sync();   // every wave's reads of the staged rows are done
#pragma unroll
    for (int it = 0; it < TRIPS; ++it) {
      if (tile[it] >= 0) {
        const int i = (tile[it] >> 8) & 255, j = tile[it] & 255;
        float* dst = (tile[it] >> 16) ? KQs : KKs;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * i + 4 * g + r) * FLD + 16 * j + li] = acc[it][r];
      }
    }
  }
  block_sync();

  // 3. L (in place of K K^T); the output mixing and the vector to the record
  E* rec = reinterpret_cast<E*>(static_cast<char*>(a.ws) + ((long)bh * a.nck + ck) * a.rec_bytes);
  E* TiT = rec;
  E* OmT = rec + CP * CP;
  float* vec = reinterpret_cast<float*>(rec + 2 * CP * CP);
  for (int e = tid; e < CP * CP; e += NTH) {
    const int t = e / CP, u = e % CP;   // consecutive threads: consecutive u
    const bool valid = u < C && t < C;
    const int fu = fr[u], ft = fr[t];
    const float kk = KKs[u * FLD + t], kq = KQs[u * FLD + t];
    KKs[u * FLD + t] = (valid && fu < ft) ? s2 * kk * Dt[dti(fu + 1, ft)] * bs[t] : 0.f;
    OmT[t * CP + u] = toE((valid && fu <= ft) ? s * kq * Dt[dti(fu + 1, ft + 1)] : 0.f);
  }
  if (tid < CP) {
    const int t = tid, f = fr[t];
    const bool valid = t < C;
    vec[t] = valid ? Dt[dti(0, f)] : 0.f;                    // P(0, f(t) - 1)
    vec[CP + t] = valid ? Dt[dti(0, f + 1)] : 0.f;           // P(0, f(t))
    vec[2 * CP + t] = valid ? Dt[dti(f + 1, nf)] : 0.f;      // P(f(t) + 1, F - 1)
    vec[3 * CP + t] = bs[t];                                 // beta_t
    vec[4 * CP + t] = t == 0 ? Dt[dti(0, nf)] : 0.f;         // P(0, F - 1)
  }
  block_sync();

  // 4. (I + L)^-1 into KQs: diagonal blocks by substitution (lane c holds
  // column c; column-oriented, so that the updates of one step are
  // independent and the dependent chain is 15 steps long, not 120), then
  // block back-substitution by distance
  for (int I = w; I < NB; I += NW) {
    if (g == 0) {
      const float* Lb = &KKs[16 * I * FLD + 16 * I];
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == li) ? 1.f : 0.f;
#pragma unroll
      for (int j = 15; j > 0; --j)
#pragma unroll
        for (int i = 0; i < j; ++i) x[i] -= Lb[i * FLD + j] * x[j];
#pragma unroll
      for (int i = 0; i < 16; ++i) KQs[(16 * I + i) * FLD + 16 * I + li] = x[i];
    }
  }
  block_sync();
  for (int d = 1; d < NB; ++d) {
    for (int I = w; I < NB - d; I += NW) {
      const int J = I + d;
      f32x4 y = zero4();
      for (int Kb = I + 1; Kb <= J; ++Kb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          y = mfma_f32(KKs[(16 * I + li) * FLD + 16 * Kb + 4 * kk + g],
                       KQs[(16 * Kb + 4 * kk + g) * FLD + 16 * J + li], y);
#pragma unroll
      for (int r = 0; r < 4; ++r) Ys[I][(4 * g + r) * 16 + li] = y[r];
      fence();
      f32x4 x = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x = mfma_f32(KQs[(16 * I + li) * FLD + 16 * I + 4 * kk + g], Ys[I][(4 * kk + g) * 16 + li], x);
#pragma unroll
      for (int r = 0; r < 4; ++r) KQs[(16 * I + 4 * g + r) * FLD + 16 * J + li] = -x[r];
    }
    block_sync();
  }
  // 5. the inverse, transposed: TiT[t][u] = (I + L)^-1[u][t]
  for (int e = tid; e < CP * CP; e += NTH) {
    const int t = e / CP, u = e % CP;
    TiT[t * CP + u] = toE((u >> 4) <= (t >> 4) ? KQs[u * FLD + t] : 0.f);
  }
}

// ---------------------------------------------------------------------------
// The state pass: one workgroup per (b, h), wave w owns state rows
// 16 w .. 16 w + 15 (in fp32 registers), chunks in order.  OUTS: the pass
// emits outputs (TOK_PLAIN, TOK_REPLAY); the composite pass does not, and
// neither loads Q and Om nor forms E_0 Q^T and W Om.
template <int IO, int NT, bool OUTS>
__global__ __launch_bounds__(64 * NT) void token_scan_kernel(TokArgs a) {
  typedef TokLayout<IO, NT> Y;
  typedef typename Y::E E;
  constexpr bool BF = Y::BF;
  constexpr int D = Y::D, CP = Y::CP, NB = Y::NB, KS = Y::KS, DP = Y::DP, PAD = Y::PAD;
  constexpr int KLD = Y::KLD, TLD = Y::TLD, PR = Y::PR, EP = Y::EP, CPR = Y::CPR;
  constexpr int ZW = DP > 2 * CP ? DP : 2 * CP;
  constexpr int ZLD = ZW + PAD;               // a wave's staged rows
  constexpr int NTH = 64 * NT;
  constexpr int VEC = 5 * CP;                 // floats of a chunk's decay/gate vector
  // ring pieces (16 bytes): K and Q rows, the two CP x CP operators, the vector
  constexpr int NKQ = 2 * CP * PR, NOP = 2 * CP * CPR, NVEC = VEC * 4 / 16;
  constexpr int NPC = NKQ + NOP + NVEC;
  constexpr int PPT = (NPC + NTH - 1) / NTH;

  __shared__ __attribute__((aligned(16))) E Ks[CP * KLD];
  __shared__ __attribute__((aligned(16))) E Qs[CP * KLD];
  __shared__ __attribute__((aligned(16))) E TiT[CP * TLD];
  __shared__ __attribute__((aligned(16))) E OmT[CP * TLD];
  __shared__ __attribute__((aligned(16))) float vec[VEC];
  __shared__ __attribute__((aligned(16))) E Zs[NT][16 * ZLD];

  // Work item: (b, h) with a.nseg == 1; else (b, h, segment) and, in the
  // composite pass, which of the two walks (input composite H from zero
  // with V, transition composite Phi from the identity without V).
  const int nwalk = a.mode == TOK_COMPOSITE ? 2 : 1;
  const int walk = blockIdx.x % nwalk;
  const int seg = (blockIdx.x / nwalk) % a.nseg;
  const int bh = blockIdx.x / nwalk / a.nseg;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const bool phi = walk == 1;               // the transition walk: no inputs, no outputs
  const int ck_beg = seg * a.cps;
  const int ck_end = min(a.nck, ck_beg + a.cps);
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, T = a.T;
  const long L = (long)T * N;
  const float s = a.s;
  const E* K = static_cast<const E*>(a.k);
  const E* Q = static_cast<const E*>(a.q);
  const E* V = static_cast<const E*>(a.v);
  E* O = static_cast<E*>(a.o);
  E* Zw = Zs[w];

  auto toE = [](float x) -> E {
    if constexpr (BF) return f32_to_bf16_bits(x); else return x;
  };
  auto fragA = [&](const E* M, int ld, int m0, int k0) {
    if constexpr (BF) return load_bf16x8(M + (m0 + li) * ld + k0 + 8 * g);
    else return M[(m0 + li) * ld + k0 + g];
  };
  auto fragBn = [&](const E* M, int ld, int k0, int n0) {
    if constexpr (BF) return lds_col_frag_bf16(M, ld, k0, n0);
    else return M[(k0 + g) * ld + n0 + li];
  };
  auto mma = [&](auto x, auto y, f32x4 c) {
    if constexpr (BF) return mfma_bf16(x, y, c); else return mfma_f32(x, y, c);
  };
  auto fence = []() {   // a wave's LDS writes land before its lanes read them back
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
  };

  // Register ring, one chunk ahead: 16-byte pieces p = tid + NTH j of
  // [K rows | Q rows | TiT, OmT | vector], and this lane's V values.
  typedef typename std::conditional<BF, u32x2, f32x4>::type VP;
  struct Pre {
    u32x4 pc[PPT];
    VP v[NB];
  };
  auto prefetch = [&](Pre& P, int ck) {
    const int t0 = ck * a.F;
    const int Cn = min(a.F, T - t0) * N;
    const long tok0 = (long)t0 * N;
    const char* rec = static_cast<const char*>(a.ws) + ((long)bh * a.nck + ck) * a.rec_bytes;
    const bool with_v = !phi;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      P.pc[j] = u32x4{0u, 0u, 0u, 0u};
      if (p < NKQ) {
        const int m = p / (CP * PR), q = p % (CP * PR), u = q / PR;
        if (u < Cn && (OUTS || m == 0))
          P.pc[j] = *reinterpret_cast<const u32x4*>(
              (m ? Q : K) + (((long)b * L + tok0 + u) * a.H + h) * D + (q % PR) * EP);
      } else if (p < NPC) {
        if (OUTS || p - NKQ < CP * CPR || p >= NKQ + NOP)   // no Om without outputs
          P.pc[j] = *reinterpret_cast<const u32x4*>(rec + (long)(p - NKQ) * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = 16 * j + li;
      P.v[j] = VP{};
      if (with_v && t < Cn)
        P.v[j] = *reinterpret_cast<const VP*>(V + (((long)b * L + tok0 + t) * a.H + h) * D +
                                               16 * w + 4 * g);
    }
  };
  auto commit = [&](const Pre& P) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      if (p < NKQ) {
        const int m = p / (CP * PR), q = p % (CP * PR);
        *reinterpret_cast<u32x4*>(&(m ? Qs : Ks)[(q / PR) * KLD + (q % PR) * EP]) = P.pc[j];
      } else if (p < NKQ + NOP) {
        const int o = p - NKQ, m = o / (CP * CPR), q = o % (CP * CPR);
        *reinterpret_cast<u32x4*>(&(m ? OmT : TiT)[(q / CPR) * TLD + (q % CPR) * EP]) = P.pc[j];
      } else if (p < NPC) {
        *reinterpret_cast<u32x4*>(&vec[(p - NKQ - NOP) * 4]) = P.pc[j];
      }
    }
  };

  // the state: wave w holds rows 16 w .. 16 w + 15, tile n in Sreg[n]
  // Entering state: the initial state (one segment), the fold's entering
  // state of the segment (replay), zero (H walk) or the identity (Phi walk).
  const float* zs = a.mode == TOK_REPLAY ? a.zin + ((long)bh * a.nseg + seg) * D * D
                  : a.mode == TOK_PLAIN && a.z0 ? a.z0 + (long)bh * D * D : nullptr;
  f32x4 Sreg[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Sreg[n][r] = zs ? zs[(16 * w + 4 * g + r) * D + 16 * n + li]
                      : (phi && 16 * w + 4 * g + r == 16 * n + li ? 1.f : 0.f);
  }
  // feature padding of K and Q rows: zero once, never written again
  if constexpr (DP > D) {
    for (int e = tid; e < CP * (DP - D); e += NTH) {
      const int u = e / (DP - D), c = D + e % (DP - D);
      Ks[u * KLD + c] = toE(0.f);
      Qs[u * KLD + c] = toE(0.f);
    }
  }

  Pre cur, nxt;
  prefetch(cur, ck_beg);
  for (int ck = ck_beg; ck < ck_end; ++ck) {
    const int t0 = ck * a.F;
    const int C = min(a.F, T - t0) * N;
    const long tok0 = (long)t0 * N;

    // 1. this chunk's inputs into LDS, the state rows staged; next chunk's
    // loads in flight
    commit(cur);
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) Zw[(4 * g + r) * ZLD + 16 * n + li] = toE(Sreg[n][r]);
    if constexpr (DP > D) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Zw[(4 * g + r) * ZLD + D + li] = toE(0.f);
    }
    if (ck + 1 < ck_end) prefetch(nxt, ck + 1);
    block_sync();

    // 2. SK = E_0 K^T, SQ = E_0 Q^T (the staged rows are the A operand of all)
    f32x4 SK[NB], SQ[NB];
    {
      decltype(fragA(Zw, ZLD, 0, 0)) af[DP / KS];
#pragma unroll
      for (int kb = 0; kb < DP / KS; ++kb) af[kb] = fragA(Zw, ZLD, 0, kb * KS);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4 sk = zero4(), sq = zero4();
#pragma unroll
        for (int kb = 0; kb < DP / KS; ++kb) {
          sk = mma(af[kb], fragA(Ks, KLD, 16 * j, kb * KS), sk);
          if constexpr (OUTS) sq = mma(af[kb], fragA(Qs, KLD, 16 * j, kb * KS), sq);
        }
        SK[j] = sk;
        SQ[j] = sq;
      }
    }
    fence();

    // 3. R = (V - P(0, f - 1) s SK) beta, staged; W = R (I + L)^-1
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = 16 * j + li;
      f32x4 vv;
      if constexpr (BF) {
        vv[0] = bf16_bits_to_f32((uint16_t)(cur.v[j][0] & 0xffff));
        vv[1] = bf16_bits_to_f32((uint16_t)(cur.v[j][0] >> 16));
        vv[2] = bf16_bits_to_f32((uint16_t)(cur.v[j][1] & 0xffff));
        vv[3] = bf16_bits_to_f32((uint16_t)(cur.v[j][1] >> 16));
      } else {
        vv = cur.v[j];
      }
      const float before = vec[t], bt = vec[3 * CP + t];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Zw[(4 * g + r) * ZLD + t] = toE((vv[r] - s * before * SK[j][r]) * bt);
    }
    fence();
    f32x4 Wr[NB];
    {
      decltype(fragA(Zw, ZLD, 0, 0)) rf[CP / KS];
#pragma unroll
      for (int kb = 0; kb < CP / KS; ++kb) rf[kb] = fragA(Zw, ZLD, 0, kb * KS);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < CP / KS; ++kb) acc = mma(rf[kb], fragA(TiT, TLD, 16 * j, kb * KS), acc);
        Wr[j] = acc;
      }
    }
    fence();

    // 4. W and W tail staged; O = P(0, f) SQ + W Om
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = 16 * j + li;
      const float tail = vec[2 * CP + t];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (OUTS) Zw[(4 * g + r) * ZLD + t] = toE(Wr[j][r]);
        Zw[(4 * g + r) * ZLD + CP + t] = toE(Wr[j][r] * tail);
      }
    }
    fence();
    if constexpr (OUTS) {
      decltype(fragA(Zw, ZLD, 0, 0)) wf[CP / KS];
#pragma unroll
      for (int kb = 0; kb < CP / KS; ++kb) wf[kb] = fragA(Zw, ZLD, 0, kb * KS);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < CP / KS; ++kb) acc = mma(wf[kb], fragA(OmT, TLD, 16 * j, kb * KS), acc);
        const int t = 16 * j + li;
        if (t < C) {
          const float upto = vec[CP + t];
          f32x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = upto * SQ[j][r] + acc[r];
          const long off = (((long)b * L + tok0 + t) * a.H + h) * D + 16 * w + 4 * g;
          if constexpr (BF) {
            u32x2 pk;
            pk[0] = (uint32_t)f32_to_bf16_bits(ov[0]) | ((uint32_t)f32_to_bf16_bits(ov[1]) << 16);
            pk[1] = (uint32_t)f32_to_bf16_bits(ov[2]) | ((uint32_t)f32_to_bf16_bits(ov[3]) << 16);
            *reinterpret_cast<u32x2*>(O + off) = pk;
          } else {
            *reinterpret_cast<f32x4*>(O + off) = ov;
          }
        }
      }
    }

    // 5. E_F = P(0, F-1) E_0 + s (W tail) K
    const float total = vec[4 * CP];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < CP / KS; ++kb)
        acc = mma(fragA(Zw + CP, ZLD, 0, kb * KS), fragBn(Ks, KLD, kb * KS, 16 * n), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) Sreg[n][r] = total * Sreg[n][r] + s * acc[r];
    }
    cur = nxt;
    block_sync();   // every wave is done with this chunk's LDS inputs
  }

  if (a.mode == TOK_COMPOSITE) {
    // H in the MFMA tile order, -Phi^T row-major: the layouts the frame
    // form's fold reads its composites in
    const long base = ((long)bh * a.nseg + seg) * D * D;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (!phi)
        *reinterpret_cast<f32x4*>(a.compH + base + ((w * NT + n) * 64 + lane) * 4) = Sreg[n];
      else
        *reinterpret_cast<f32x4*>(a.compC + base + (16 * n + li) * D + 16 * w + 4 * g) = -Sreg[n];
    }
  } else if (a.zT && seg == a.nseg - 1) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.zT[((long)bh * D + 16 * w + 4 * g + r) * D + 16 * n + li] = Sreg[n][r];
  }
}

template <int IO>
static hipError_t launch_token_io(const TokArgs& a, int nt, bool prep, hipStream_t s) {
  const dim3 pgrid(a.B * a.H * a.nck), pblock(512);
  const dim3 sgrid(a.B * a.H * a.nseg * (a.mode == TOK_COMPOSITE ? 2 : 1)), sblock(64 * nt);
  switch (nt) {
#define GDN_TOK_CASE(n)                                                               \
  case n:                                                                             \
    if (prep) hipLaunchKernelGGL((token_prep_kernel<IO, n>), pgrid, pblock, 0, s, a); \
    if (a.mode == TOK_COMPOSITE)                                                       \
      hipLaunchKernelGGL((token_scan_kernel<IO, n, false>), sgrid, sblock, 0, s, a);  \
    else                                                                               \
      hipLaunchKernelGGL((token_scan_kernel<IO, n, true>), sgrid, sblock, 0, s, a);   \
    break;
    GDN_TOK_CASE(1) GDN_TOK_CASE(2) GDN_TOK_CASE(3) GDN_TOK_CASE(4)
    GDN_TOK_CASE(5) GDN_TOK_CASE(6) GDN_TOK_CASE(7) GDN_TOK_CASE(8)
#undef GDN_TOK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_token(const TokArgs& a, int io, int nt, bool prep, hipStream_t s) {
  const int cp = io == IO_BF16 ? TokCfg<IO_BF16>::CP : TokCfg<IO_F32>::CP;
  if (a.N < 1 || a.F < 1 || a.F * a.N > cp || a.nck != (a.T + a.F - 1) / a.F ||
      a.rec_bytes != token_record_bytes(io) || !a.ws || a.nseg < 1 || a.cps < 1 ||
      (long)a.nseg * a.cps < a.nck || (long)(a.nseg - 1) * a.cps >= a.nck ||
      (a.mode == TOK_COMPOSITE && (!a.compH || !a.compC)) || (a.mode == TOK_REPLAY && !a.zin) ||
      (a.mode == TOK_PLAIN && a.nseg != 1))
    return hipErrorInvalidValue;
  return io == IO_BF16 ? launch_token_io<IO_BF16>(a, nt, prep, s)
                       : launch_token_io<IO_F32>(a, nt, prep, s);
}

}  // namespace gdn
