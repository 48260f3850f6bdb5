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
// each other), so I + L is unit upper triangular: its inverse is formed per
// chunk by substitution on the 16 x 16 diagonal blocks and block
// back-substitution above them (fp32), and W = R (I + L)^-1.
//
// One workgroup per (b, h) sequence, one wave per 16 state rows (rows of S
// evolve independently); the token x token products of a chunk (K K^T,
// K Q^T, the triangular inverse) are shared by the waves through LDS.
// bf16 io: bf16 MFMA 16x16x32 with fp32 accumulation, the state and the
// corrected values rounded to bf16 as MFMA operands (as in the frame form's
// scan); fp32 io: fp32 MFMA 16x16x4 throughout.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int IO, int NT>
__global__ __launch_bounds__(64 * NT) void token_kernel(TokArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr int D = 16 * NT;
  constexpr int CP = TokCfg<IO>::CP;          // tokens per chunk at most
  constexpr int NB = CP / 16;                 // 16-token blocks
  constexpr int KS = BF ? 32 : 4;             // MFMA contraction depth
  constexpr int DP = (D + KS - 1) / KS * KS;  // feature dim padded to KS (zeros)
  constexpr int PAD = BF ? 8 : 4;             // 16 bytes
  constexpr int KLD = DP + PAD;               // K, Q rows in LDS
  constexpr int ZW = DP > 2 * CP ? DP : 2 * CP;
  constexpr int ZLD = ZW + PAD;               // a wave's staged rows
  constexpr int FLD = CP + 1;                 // fp32 token x token matrices
  constexpr int TLD = CP + PAD;               // their transposed MFMA copies
  constexpr int DLD = CP + 1;                 // decay table
  constexpr int NTH = 64 * NT;
  constexpr int PR = D * Io<IO>::bytes / 16;  // 16-byte pieces of a token row
  constexpr int EP = 16 / Io<IO>::bytes;      // elements per piece

  __shared__ __attribute__((aligned(16))) E Ks[CP * KLD];
  __shared__ __attribute__((aligned(16))) E Qs[CP * KLD];
  __shared__ __attribute__((aligned(16))) E Zs[NT][16 * ZLD];
  __shared__ float KKs[CP * FLD];      // K^ K^^T, then L in place
  __shared__ float KQs[CP * FLD];      // K Q^T, then (I + L)^-1
  __shared__ __attribute__((aligned(16))) E TiT[CP * TLD];   // (I + L)^-1, transposed
  __shared__ __attribute__((aligned(16))) E OmT[CP * TLD];   // output mixing, transposed
  __shared__ float Dt[(CP + 1) * DLD];  // Dt[x][c] = P(x, c - 1)
  __shared__ float Ys[NB][256];
  __shared__ float gs[CP], bs[CP];

  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N, T = a.T;
  const long L = (long)T * N;
  const float s = a.s, s2 = a.s * a.s;
  const E* K = static_cast<const E*>(a.k);
  const E* Q = static_cast<const E*>(a.q);
  const E* V = static_cast<const E*>(a.v);
  E* O = static_cast<E*>(a.o);
  E* Zw = Zs[w];

  auto toE = [](float x) -> E {
    if constexpr (BF) return f32_to_bf16_bits(x); else return x;
  };
  // MFMA operands.  A[m][k] = M[m0 + m][k0 + k]; Bt: B[k][n] = M[n0 + n][k0 + k];
  // Bn: B[k][n] = M[k0 + k][n0 + n] (M row-major with row stride ld).
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
  // 16 x 16 tile of (rows of A) x (rows of Bm)^T over kn contraction steps
  auto tile_nt = [&](const E* Am, int lda, int m0, const E* Bm, int ldb, int n0, int kn) {
    f32x4 acc = zero4();
    for (int kb = 0; kb < kn; ++kb) acc = mma(fragA(Am, lda, m0, kb * KS), fragA(Bm, ldb, n0, kb * KS), acc);
    return acc;
  };
  // a wave's own LDS writes complete before it reads them back in other lanes
  auto fence = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
  };

  // the state: wave w holds rows 16 w .. 16 w + 15, tile n in Sreg[n]
  f32x4 Sreg[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    Sreg[n] = zero4();
    if (a.z0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Sreg[n][r] = a.z0[((long)bh * D + 16 * w + 4 * g + r) * D + 16 * n + li];
    }
  }
  // zero feature padding of K and Q rows once (never written again)
  if constexpr (DP > D) {
    for (int e = tid; e < CP * (DP - D); e += NTH) {
      const int u = e / (DP - D), c = D + e % (DP - D);
      Ks[u * KLD + c] = toE(0.f);
      Qs[u * KLD + c] = toE(0.f);
    }
  }

  for (int t0 = 0; t0 < T; t0 += a.F) {
    const int nf = min(a.F, T - t0);
    const int C = nf * N;
    const long tok0 = (long)t0 * N;

    // 1. the chunk's K, Q rows (zero past C), gates, and this wave's state rows
    for (int p = tid; p < CP * PR; p += NTH) {
      const int u = p / PR, c = (p % PR) * EP;
      u32x4 kv = u32x4{0u, 0u, 0u, 0u}, qv = kv;
      if (u < C) {
        const long off = (((long)b * L + tok0 + u) * a.H + h) * D + c;
        kv = *reinterpret_cast<const u32x4*>(K + off);
        qv = *reinterpret_cast<const u32x4*>(Q + off);
      }
      *reinterpret_cast<u32x4*>(&Ks[u * KLD + c]) = kv;
      *reinterpret_cast<u32x4*>(&Qs[u * KLD + c]) = qv;
    }
    if (tid < CP) {
      gs[tid] = tid < nf ? a.gamma[((long)b * T + t0 + tid) * a.H + h] : 0.f;
      bs[tid] = tid < C ? a.beta[((long)b * L + tok0 + tid) * a.H + h] : 0.f;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) Zw[(4 * g + r) * ZLD + 16 * n + li] = toE(Sreg[n][r]);
    if constexpr (DP > D) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Zw[(4 * g + r) * ZLD + D + li] = toE(0.f);
    }
    block_sync();

    // 2. decay table; token x token products; this wave's E_0 K^T and E_0 Q^T
    for (int x = tid; x <= nf; x += NTH) {
      float p = 1.f;
      Dt[x * DLD + x] = 1.f;
      for (int c = x + 1; c <= nf; ++c) {
        p *= gs[c - 1];
        Dt[x * DLD + c] = p;
      }
    }
    {
      constexpr int NP = NB * (NB + 1) / 2;   // K K^T: blocks i <= j
      for (int q = w; q < NP + NB * NB; q += NT) {
        int i, j;
        const bool kq = q >= NP;
        if (kq) {
          i = (q - NP) / NB; j = (q - NP) % NB;
        } else {
          int rem = q; i = 0;
          while (rem >= NB - i) { rem -= NB - i; ++i; }
          j = i + rem;
        }
        const f32x4 acc = tile_nt(Ks, KLD, 16 * i, kq ? Qs : Ks, KLD, 16 * j, DP / KS);
        float* dst = kq ? KQs : KKs;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * i + 4 * g + r) * FLD + 16 * j + li] = acc[r];
      }
    }
    f32x4 SK[NB], SQ[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      SK[j] = tile_nt(Zw, ZLD, 0, Ks, KLD, 16 * j, DP / KS);
      SQ[j] = tile_nt(Zw, ZLD, 0, Qs, KLD, 16 * j, DP / KS);
    }
    block_sync();

    // 3. L (in place of K K^T) and the output mixing Om (transposed copy)
    for (int e = tid; e < CP * CP; e += NTH) {
      const int u = e / CP, t = e % CP;
      const bool valid = u < C && t < C;
      const int fu = u / N, ft = t / N;
      const float kk = KKs[u * FLD + t], kq = KQs[u * FLD + t];
      KKs[u * FLD + t] = (valid && fu < ft) ? s2 * kk * Dt[(fu + 1) * DLD + ft] * bs[t] : 0.f;
      OmT[t * TLD + u] = toE((valid && fu <= ft) ? s * kq * Dt[(fu + 1) * DLD + ft + 1] : 0.f);
    }
    block_sync();

    // 4. (I + L)^-1 into KQs: diagonal blocks by substitution (lane c of
    // the wave handling block I holds column c), then block
    // back-substitution by distance; blocks are dealt to the waves in turn
    for (int I = w; I < NB; I += NT) {
      if (g == 0) {
        const float* Lb = &KKs[16 * I * FLD + 16 * I];
        float x[16];
#pragma unroll
        for (int i = 15; i >= 0; --i) {
          float acc = (i == li) ? 1.f : 0.f;
#pragma unroll
          for (int j = i + 1; j < 16; ++j) acc -= Lb[i * FLD + j] * x[j];
          x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) KQs[(16 * I + i) * FLD + 16 * I + li] = x[i];
      }
    }
    block_sync();
    for (int d = 1; d < NB; ++d) {
      for (int I = w; I < NB - d; I += NT) {
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
    for (int e = tid; e < CP * CP; e += NTH) {
      const int u = e / CP, t = e % CP;
      TiT[t * TLD + u] = toE((u >> 4) <= (t >> 4) ? KQs[u * FLD + t] : 0.f);
    }
    block_sync();

    // 5. R for this wave's rows, then W = R (I + L)^-1
    f32x4 Wr[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = 16 * j + li;
      f32x4 vv = zero4();
      if (t < C) {
        const long off = (((long)b * L + tok0 + t) * a.H + h) * D + 16 * w + 4 * g;
        if constexpr (BF) {
          const u32x2 pv = *reinterpret_cast<const u32x2*>(V + off);
          vv[0] = bf16_bits_to_f32((uint16_t)(pv[0] & 0xffff));
          vv[1] = bf16_bits_to_f32((uint16_t)(pv[0] >> 16));
          vv[2] = bf16_bits_to_f32((uint16_t)(pv[1] & 0xffff));
          vv[3] = bf16_bits_to_f32((uint16_t)(pv[1] >> 16));
        } else {
          vv = *reinterpret_cast<const f32x4*>(V + off);
        }
      }
      const float before = t < C ? Dt[t / N] : 0.f;   // P(0, f(t) - 1)
      const float bt = bs[t];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Zw[(4 * g + r) * ZLD + t] = toE((vv[r] - s * before * SK[j][r]) * bt);
    }
    fence();
#pragma unroll
    for (int j = 0; j < NB; ++j) Wr[j] = tile_nt(Zw, ZLD, 0, TiT, TLD, 16 * j, CP / KS);
    fence();

    // 6. outputs: O = P(0, f(t)) E_0 Q + W Om
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = 16 * j + li;
      const float tail = t < C ? Dt[(t / N + 1) * DLD + nf] : 0.f;   // P(f(t)+1, F-1)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Zw[(4 * g + r) * ZLD + t] = toE(Wr[j][r]);
        Zw[(4 * g + r) * ZLD + CP + t] = toE(Wr[j][r] * tail);
      }
    }
    fence();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const f32x4 acc = tile_nt(Zw, ZLD, 0, OmT, TLD, 16 * j, CP / KS);
      const int t = 16 * j + li;
      if (t < C) {
        const float upto = Dt[t / N + 1];   // P(0, f(t))
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

    // 7. E_F = P(0, F-1) E_0 + (W tail) K^
    const float total = Dt[nf];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f32x4 acc = zero4();
      for (int kb = 0; kb < CP / KS; ++kb)
        acc = mma(fragA(Zw + CP, ZLD, 0, kb * KS), fragBn(Ks, KLD, kb * KS, 16 * n), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) Sreg[n][r] = total * Sreg[n][r] + s * acc[r];
    }
    block_sync();
  }

  if (a.zT) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.zT[((long)bh * D + 16 * w + 4 * g + r) * D + 16 * n + li] = Sreg[n][r];
  }
}

template <int IO>
static hipError_t launch_token_io(const TokArgs& a, int nt, hipStream_t s) {
  const dim3 grid(a.B * a.H), block(64 * nt);
  switch (nt) {
#define GDN_TOK_CASE(n) \
  case n: hipLaunchKernelGGL((token_kernel<IO, n>), grid, block, 0, s, a); break;
    GDN_TOK_CASE(1) GDN_TOK_CASE(2) GDN_TOK_CASE(3) GDN_TOK_CASE(4)
    GDN_TOK_CASE(5) GDN_TOK_CASE(6) GDN_TOK_CASE(7) GDN_TOK_CASE(8)
#undef GDN_TOK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_token(const TokArgs& a, int io, int nt, hipStream_t s) {
  if (a.N < 1 || a.F < 1 || a.F * a.N > (io == IO_BF16 ? TokCfg<IO_BF16>::CP : TokCfg<IO_F32>::CP))
    return hipErrorInvalidValue;
  return io == IO_BF16 ? launch_token_io<IO_BF16>(a, nt, s) : launch_token_io<IO_F32>(a, nt, s);
}

}  // namespace gdn
