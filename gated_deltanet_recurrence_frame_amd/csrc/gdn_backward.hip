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
// dQ = S_t^T dO is the output kernel run on S_t^T (gdn_output.hip).
// bwd_kv_kernel: one workgroup per frame, one wave per 16-feature tile.
// Each wave keeps its rows of G_t, G_t^T and W_t as MFMA operands in
// registers; K, V and beta are copied straight into a 3-stage LDS ring in
// 32-token chunks, dK and dV rows are staged in LDS and stored one chunk
// later as contiguous 16-byte pieces.  dbeta sums the per-feature-tile
// partial dot products in a fixed order (deterministic, no atomics).
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

template <int IO, int NT>
__global__ __launch_bounds__(64 * NT) void bwd_kv_kernel(BwdTokArgs a) {
  typedef typename Io<IO>::elem E;
  constexpr bool BF = (IO == IO_BF16);
  constexpr int D = 16 * NT;
  constexpr int ES = Io<IO>::bytes;
  constexpr int CT = 32;                          // tokens per chunk
  constexpr int MAT_BYTES = CT * D * ES;          // one chunk of K (or V) rows
  constexpr int WL = MAT_BYTES / 1024;            // 1 KB copies per matrix (NT or 2 NT)
  constexpr int OPS = WL / NT;                    // per wave per matrix
  constexpr int STAGE_BYTES = 2 * MAT_BYTES + 256;   // K, V, beta
  constexpr int STAGES = BF ? 3 : 2;              // fp32 rows are twice as large
  constexpr int NTH = 64 * NT;
  constexpr int KB = BF ? (D + 31) / 32 : D / 4;
  static_assert(WL % NT == 0, "copies must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char ring[STAGES][STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) E obuf[2][2][CT * D];   // dK, dV staging
  __shared__ float red[2][NT][CT];                               // dbeta partials

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

  // Left operands of this wave's feature tile: rows of G_t, of G_t^T
  // (columns of G_t, staged in LDS and read with the transposing read) and
  // of W_t (symmetric).
  const E* Gt = static_cast<const E*>(a.G) + moff;
  const E* Wt = static_cast<const E*>(a.W) + moff;
  const int fr = ft * 16 + li;
  typedef typename std::conditional<BF, bf16x8, float>::type Frag;
  Frag mG[KB], mGT[KB], mW[KB];
  if constexpr (BF) {
    uint16_t* ms = reinterpret_cast<uint16_t*>(&obuf[0][0][0]);   // [KB*32][D], 4 KB * NT * 2
    static_assert(KB * 32 * D * 2 <= 2 * 2 * CT * D * 2, "staging fits");
    constexpr int PRW = D / 8;
    for (int p = tid; p < KB * 32 * PRW; p += NTH) {
      const int row = p / PRW, pc = p % PRW;
      *reinterpret_cast<u32x4*>(ms + row * D + pc * 8) =
          row < D ? *reinterpret_cast<const u32x4*>(Gt + row * D + pc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    block_sync();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 32 + 8 * g;
      mGT[kb] = lds_col_frag_bf16(ms, D, kb * 32, ft * 16);
      mG[kb] = (k < D) ? load_bf16x8(Gt + fr * D + k) : zero_bf16x8();
      mW[kb] = (k < D) ? load_bf16x8(Wt + fr * D + k) : zero_bf16x8();
    }
    block_sync();
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = kb * 4 + g;
      mG[kb] = Gt[fr * D + k];
      mGT[kb] = Gt[k * D + fr];
      mW[kb] = Wt[fr * D + k];
    }
  }

  // Copies of a chunk: K pieces (op i < WL), V pieces (WL <= i < 2 WL), 1 KB
  // each, lane l's 16 bytes at + 16 l; wave 0 also copies the chunk's beta.
  const char* ksrc = static_cast<const char*>(a.k);
  const char* vsrc = static_cast<const char*>(a.v);
  auto issue = [&](int c) {
    const int c0 = c * CT;
    char* st = ring[c % STAGES];
#pragma unroll
    for (int j = 0; j < 2 * OPS; ++j) {
      const int i = ft + NT * j;
      const int m = i / WL, w = i % WL;
      const int o = w * 1024 + lane * 16;
      const int row = o / (D * ES), col = o % (D * ES);
      int tk = c0 + row;
      if (tk >= N) tk = N - 1;
      dma16((m ? vsrc : ksrc) + (((row0 + tk) * a.H + h) * (long)D) * ES + col,
            st + m * MAT_BYTES + w * 1024);
    }
    if (ft == 0) {
      int tk = c0 + lane;
      if (tk >= N) tk = N - 1;          // lanes past the chunk or the frame: unused
      dma4(a.beta + (row0 + tk) * a.H + h, st + 2 * MAT_BYTES);
    }
  };
  auto store_chunk = [&](int c) {
    constexpr int PRW = D * ES / 16;
    for (int p = tid; p < 2 * CT * PRW; p += NTH) {
      const int m = p / (CT * PRW), r = p % (CT * PRW);
      const int row = r / PRW, pc = r % PRW;
      const int tk = c * CT + row;
      if (tk < N)
        *reinterpret_cast<u32x4*>(static_cast<E*>(m ? a.dv : a.dk) +
                                  ((row0 + tk) * a.H + h) * (long)D + pc * (16 / ES)) =
            *reinterpret_cast<const u32x4*>(&obuf[c & 1][m][row * D + pc * (16 / ES)]);
    }
    if (tid < CT) {
      const int tk = c * CT + tid;
      if (tk < N) {
        float sum = 0.f;
#pragma unroll
        for (int f = 0; f < NT; ++f) sum += red[c & 1][f][tid];
        a.dbeta[(row0 + tk) * a.H + h] = sum;
      }
    }
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

  const int nchunks = (N + CT - 1) / CT;
#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c)
    if (c < nchunks) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    // with 3 stages chunk c+1's copies (2 OPS per wave, at least) are
    // younger than chunk c's; with 2 stages nothing younger is in flight
    if (STAGES == 3 && c + 1 < nchunks)
      wait_vm_barrier<2 * OPS>();
    else
      wait_vm_barrier<0>();
    if (c + STAGES - 1 < nchunks) issue(c + STAGES - 1);
    if (c > 0) store_chunk(c - 1);
    const char* st = ring[c % STAGES];
    const E* ks = reinterpret_cast<const E*>(st);
    const E* vs = reinterpret_cast<const E*>(st + MAT_BYTES);
    const float* bs = reinterpret_cast<const float*>(st + 2 * MAT_BYTES);
#pragma unroll
    for (int tt = 0; tt < CT / 16; ++tt) {
      const int trow = tt * 16 + li;
      f32x4 ay = zero4(), az = zero4(), aw = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (BF) {
          const int k = kb * 32 + 8 * g;
          const bool ok = k < D;
          const bf16x8 kf = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(ks + trow * D) + k)
                               : zero_bf16x8();
          const bf16x8 vf = ok ? load_bf16x8(reinterpret_cast<const uint16_t*>(vs + trow * D) + k)
                               : zero_bf16x8();
          ay = mfma_bf16(mG[kb], kf, ay);
          az = mfma_bf16(mGT[kb], vf, az);
          aw = mfma_bf16(mW[kb], kf, aw);
        } else {
          const int k = kb * 4 + g;
          const float kf = reinterpret_cast<const float*>(ks)[trow * D + k];
          const float vf = reinterpret_cast<const float*>(vs)[trow * D + k];
          ay = mfma_f32(mG[kb], kf, ay);
          az = mfma_f32(mGT[kb], vf, az);
          aw = mfma_f32(mW[kb], kf, aw);
        }
      }
      const float bt = (c * CT + trow < N) ? bs[trow] : 0.f;
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
      if (g == 0) red[c & 1][ft][trow] = part;
      put4(&obuf[c & 1][0][trow * D + ft * 16 + 4 * g], dkv);
      put4(&obuf[c & 1][1][trow * D + ft * 16 + 4 * g], dvv);
    }
  }
  block_sync();
  store_chunk(nchunks - 1);
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
  hipLaunchKernelGGL((bwd_kv_kernel<IO, NT>), dim3(a.B * a.T * a.H), dim3(64 * NT), 0, s, a);
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
