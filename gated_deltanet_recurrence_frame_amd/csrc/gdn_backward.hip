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
// dm_kernel: one workgroup per frame forms dM_t on MFMA from S_{t-1} and G_t
// staged in LDS (bf16: both operands read with the transposing LDS read;
// fp32: 16x16x4 fp32 MFMA), writes W_t and dgamma_t (a fixed-order block
// sum).
// bwd_tok_kernel: one workgroup per frame, one wave per 16-feature tile.
// Each wave keeps its rows of S_t^T, G_t, G_t^T and W_t as MFMA operands
// in registers; K, V, dO and beta stream through LDS in token chunks.  The
// per-token dbeta sums partial dot products over the feature tiles in a
// fixed order (deterministic, no atomics).
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
  for (int idx = tid; idx < KP * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    float sv = 0.f, gv = 0.f;
    if (i < D) {
      gv = BF ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(Gt)[idx])
              : reinterpret_cast<const float*>(Gt)[idx];
      if (Sp)
        sv = BF ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(Sp)[idx])
                : reinterpret_cast<const float*>(Sp)[idx];
      else if (S0)
        sv = BF ? bf16_bits_to_f32(f32_to_bf16_bits(S0[idx])) : S0[idx];
    }
    if constexpr (BF) {
      reinterpret_cast<uint16_t*>(Sl)[i * SLD + j] = f32_to_bf16_bits(sv);
      reinterpret_cast<uint16_t*>(Gl)[i * SLD + j] = f32_to_bf16_bits(gv);
    } else {
      reinterpret_cast<float*>(Sl)[i * SLD + j] = sv;
      reinterpret_cast<float*>(Gl)[i * SLD + j] = gv;
    }
    dot += sv * gv;
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
  for (int idx = tid; idx < D * D; idx += 256) {
    const int j = idx / D, l = idx % D;
    const float w = dm[j * LD + l] + dm[l * LD + j];
    if constexpr (BF)
      reinterpret_cast<uint16_t*>(Wt)[idx] = f32_to_bf16_bits(w);
    else
      reinterpret_cast<float*>(Wt)[idx] = w;
  }
}

template <int IO, int NT>
__global__ __launch_bounds__(64 * NT) void bwd_tok_kernel(BwdTokArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int CT = (IO == IO_BF16) ? 64 : 32;
  constexpr int PR = D * ES / 16;
  constexpr int MAT_ELEMS = CT * D;
  constexpr int PIECES = 3 * CT * PR;
  constexpr int NTH = 64 * NT;
  constexpr int PPT = (PIECES + NTH - 1) / NTH;
  constexpr int KB = (IO == IO_BF16) ? (D + 31) / 32 : D / 4;
  constexpr int STAGE_BYTES = 3 * MAT_ELEMS * ES + CT * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  __shared__ float red[NT][CT];

  const int total = a.B * a.T * a.H;
  const int item = xcd_item(blockIdx.x, total);
  const int h = item % a.H;
  const int t = (item / a.H) % a.T;
  const int b = item / (a.H * a.T);
  const int N = a.N;
  const long row0 = (long)b * a.T * N + (long)t * N;
  const long DD = (long)D * D;
  const long moff = (((long)b * a.H + h) * a.T + t) * DD;
  const int tid = threadIdx.x;
  const int lane = lane_id(), ft = wave_id();
  const int g = lane >> 4, li = lane & 15;
  const float s = a.s;

  // Operand rows of this wave's feature tile: S_t^T, G, G^T, W
  // (intermediate type, row-major in memory).
  const E* St = static_cast<const E*>(a.S) + moff;
  const E* Gt = static_cast<const E*>(a.G) + moff;
  const E* Wt = static_cast<const E*>(a.W) + moff;
  const int fr = ft * 16 + li;
  typedef typename std::conditional<IO == IO_BF16, bf16x8, float>::type Frag;
  Frag mS[KB], mG[KB], mGT[KB], mW[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if constexpr (IO == IO_BF16) {
      const int k = kb * 32 + 8 * g;
      if (k < D) {
        i16x8 vs, vgt;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vs[e] = (short)St[(k + e) * D + fr];
          vgt[e] = (short)Gt[(k + e) * D + fr];
        }
        mS[kb] = __builtin_bit_cast(bf16x8, vs);
        mGT[kb] = __builtin_bit_cast(bf16x8, vgt);
        mG[kb] = load_bf16x8(Gt + fr * D + k);
        mW[kb] = load_bf16x8(Wt + fr * D + k);
      } else {
        mS[kb] = mG[kb] = mGT[kb] = mW[kb] = zero_bf16x8();
      }
    } else {
      const int k = kb * 4 + g;
      mS[kb] = St[k * D + fr];
      mG[kb] = Gt[fr * D + k];
      mGT[kb] = Gt[k * D + fr];
      mW[kb] = Wt[fr * D + k];
    }
  }

  const E* srcs[3] = {static_cast<const E*>(a.k), static_cast<const E*>(a.v),
                      static_cast<const E*>(a.d_o)};
  u32x4 pre[PPT];
  float bpre = 0.f;
  auto issue = [&](int c) {
    const int c0 = c * CT;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      if (p < PIECES) {
        const int m = p / (CT * PR);
        const int r = p % (CT * PR);
        const int row = r / PR, pc = r % PR;
        int tk = c0 + row;
        if (tk >= N) tk = N - 1;
        pre[j] = *reinterpret_cast<const u32x4*>(srcs[m] + ((row0 + tk) * a.H + h) * (long)D +
                                                 pc * (16 / ES));
      }
    }
    if (tid < CT) {
      const int tk = c0 + tid;
      bpre = tk < N ? a.beta[(row0 + tk) * a.H + h] : 0.f;
    }
  };
  auto commit = [&](int stage) {
    char* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int p = tid + NTH * j;
      if (p < PIECES) {
        const int m = p / (CT * PR);
        const int r = p % (CT * PR);
        *reinterpret_cast<u32x4*>(reinterpret_cast<E*>(base) + m * MAT_ELEMS + r * (16 / ES)) =
            pre[j];
      }
    }
    if (tid < CT) reinterpret_cast<float*>(base + 3 * MAT_ELEMS * ES)[tid] = bpre;
  };

  auto store4 = [&](void* base, long tokrow, const f32x4& v) {
    E* dst = static_cast<E*>(base) + (tokrow * a.H + h) * (long)D + ft * 16 + 4 * g;
    if constexpr (IO == IO_BF16) {
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
      *reinterpret_cast<f32x4*>(dst) = v;
    }
  };
  auto load4 = [&](const E* row) -> f32x4 {  // 4 consecutive values at this lane's features
    f32x4 r;
    if constexpr (IO == IO_BF16) {
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

  const int nchunks = (N + CT - 1) / CT;
  issue(0);
  commit(0);
  block_sync();
  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) issue(c + 1);
    const char* base = smem + (c & 1) * STAGE_BYTES;
    const E* ks = reinterpret_cast<const E*>(base);
    const E* vs = ks + MAT_ELEMS;
    const E* os = ks + 2 * MAT_ELEMS;
    const float* bs = reinterpret_cast<const float*>(base + 3 * MAT_ELEMS * ES);
#pragma unroll 1
    for (int tt = 0; tt < CT / 16; ++tt) {
      const int trow = tt * 16 + li;
      f32x4 aq = zero4(), ay = zero4(), az = zero4(), aw = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (IO == IO_BF16) {
          const int k = kb * 32 + 8 * g;
          const bool ok = k < D;
          const bf16x8 kf = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(ks + trow * D) + k)
                               : zero_bf16x8();
          const bf16x8 vf = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(vs + trow * D) + k)
                               : zero_bf16x8();
          const bf16x8 of = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(os + trow * D) + k)
                               : zero_bf16x8();
          aq = mfma_bf16(mS[kb], of, aq);
          ay = mfma_bf16(mG[kb], kf, ay);
          az = mfma_bf16(mGT[kb], vf, az);
          aw = mfma_bf16(mW[kb], kf, aw);
        } else {
          const int k = kb * 4 + g;
          const float kf = reinterpret_cast<const float*>(ks)[trow * D + k];
          const float vf = reinterpret_cast<const float*>(vs)[trow * D + k];
          const float of = reinterpret_cast<const float*>(os)[trow * D + k];
          aq = mfma_f32(mS[kb], of, aq);
          ay = mfma_f32(mG[kb], kf, ay);
          az = mfma_f32(mGT[kb], vf, az);
          aw = mfma_f32(mW[kb], kf, aw);
        }
      }
      const float bt = bs[trow];
      const f32x4 kv = load4(ks + trow * D);
      const f32x4 vv = load4(vs + trow * D);
      f32x4 dvv, dkv;
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = s * ay[r];          // (G k^)_f
        const float w = s * aw[r];          // (W k^)_f
        dvv[r] = bt * y;
        dkv[r] = s * bt * (az[r] - w);
        part += vv[r] * y - 0.5f * s * kv[r] * w;
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (g == 0) red[ft][trow] = part;
      const int tk = c * CT + trow;
      if (tk < N) {
        store4(a.dq, row0 + tk, aq);
        store4(a.dv, row0 + tk, dvv);
        store4(a.dk, row0 + tk, dkv);
      }
    }
    block_sync();
    if (tid < CT) {
      const int tk = c * CT + tid;
      if (tk < N) {
        float sum = 0.f;
#pragma unroll
        for (int f = 0; f < NT; ++f) sum += red[f][tid];
        a.dbeta[(row0 + tk) * a.H + h] = sum;
      }
    }
    if (c + 1 < nchunks) commit((c + 1) & 1);
    block_sync();
  }
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

template <int IO, int NT>
static hipError_t launch_bwd_tok_nt(const BwdTokArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_tok_kernel<IO, NT>), dim3(a.B * a.T * a.H), dim3(64 * NT), 0, s, a);
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
