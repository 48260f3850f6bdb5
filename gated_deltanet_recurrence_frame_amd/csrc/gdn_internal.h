// Kernel argument blocks and launchers shared between the libgdn kernels and
// the host-side C ABI (gdn_api.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"   // IoKind

namespace gdn {

// Per-frame D x D intermediates are stored in the "intermediate type": bf16
// when the io dtype is bf16, fp32 when it is fp32.  Three layouts:
//   row-major  [D][D];
//   tiles      [D/16][D/16][64][4]: 16x16 tile (I, J), lane (g, i) holds
//              the elements [16 I + 4 g + r][16 J + i], r = 0..3 (the MFMA
//              accumulator layout, so a consumer in the same layout reads
//              4 contiguous values per lane);
//   fragments  (bf16 only) the bf16 MFMA operand order of 16-row blocks:
//              element [R][C] at frag_index(R, C, D), so that the 64 lanes
//              of a wave reading rows 16 I .. + 15, columns 32 k .. + 31 as
//              an operand (lane (g, i): row 16 I + i, columns 32 k + 8 g ..
//              + 7) read one contiguous 1 KB piece (512 B for the last,
//              16-column block when D % 32 == 16).  Same size as row-major.
enum MatLayout { LAYOUT_ROWMAJOR = 0, LAYOUT_TILES = 1, LAYOUT_FRAG = 2 };
__host__ __device__ inline long frag_index(int R, int C, int D) {
  return (long)(R >> 4) * 16 * D + (C >> 5) * 512 + ((((C & 31) >> 3) << 4) + (R & 15)) * 8 +
         (C & 7);
}

// Token contraction C_r = scale_r X_r^T diag(w) Y per (b, t, h) frame.
struct GramArgs {
  const void* x0;      // [B, L, H, D] io dtype
  const void* x1;      // second row operand (NR == 2) or unused
  const void* y;       // column operand (NR == 1); NR == 2 uses x0
  const float* w;      // [B, L, H] per-token weights, or nullptr for 1
  void* out0;          // [B, H, T] x D x D, intermediate type, layout0
  void* out1;          // [B, H, T] x D x D, intermediate type, layout1 (NR == 2)
  int layout0, layout1;
  float scale0, scale1;
  int B, H, T, N;
  int t0, Tc;          // frames t0 .. t0 + Tc - 1 of the T-frame tensors
  // Token splits: P > 1 splits each frame's token chunks over P workgroups,
  // which write fp32 partial sums (scaled, tile layout) to
  //   part[(((p * B + b) * H + h) * Tc + (t - t0)) * NR + r] x D x D;
  // launch_gram_reduce then sums them in a fixed order into out0 / out1.
  int P;
  float* part;
  // Normalised keys (NR == 2, Y == X_0 == K, X_1 == V): every token's key
  // row is taken as k / |k| (a zero row stays zero), normalised as it is
  // staged.
  int norm;
};
hipError_t launch_gram(const GramArgs& a, int io, int nt, int nr, hipStream_t s);
hipError_t launch_gram_reduce(const GramArgs& a, int io, int nt, int nr, hipStream_t s);

// Inter-frame scan over the carried D x D matrix Z, 16 rows per workgroup.
//   forward  (SCAN_FWD), t = t0..t0+Tc-1:   Z <- gamma_t Z - Z A_t + U_t; emit Z
//   backward (SCAN_REV), t = t0+Tc-1..t0:   Z <- Z + U_t; emit Z;
//                                           Z <- gamma_t Z - Z A_t
// z0 / zT: [B, H, D, D] fp32 initial / final Z (nullptr: zero / not written).
// gamma == nullptr means gamma_t = 0 (used by the chunk fold below).
//
// Composite (chunked) scan.  With chunk = c > 0 the walk (in walk order:
// forward or backward in t) is cut into nck = ceil(Tc / c) chunks that run
// in parallel:
//   SCAN_COMP_FWD / SCAN_COMP_REV walk each chunk w twice at once, from
//     Z = 0 with the inputs (H_w) and from Z = I without them (C_w, the
//     product of the chunk's transition matrices in walk order), and store
//     compH[w] = H_w (tiles) and compC[w] = -C_w^T (row-major), fp32;
//   a fold, the forward scan in fp32 with A = compC, U = compH,
//     gamma = nullptr and emit_entry = 1 over the nck - 1 first slots,
//     gives the state entering every chunk, Z_w = Z_{w-1} C_{w-1} + H_{w-1};
//   SCAN_FWD / SCAN_REV with the same chunk then replay every chunk from
//     zmid[w] = Z_w (slot w of [B, H, nck] x D x D fp32), emitting as the
//     sequential walk does; only the last chunk writes zT.
enum ScanMode { SCAN_FWD = 0, SCAN_REV = 1, SCAN_COMP_FWD = 2, SCAN_COMP_REV = 3 };
struct ScanArgs {
  const void* A;        // [B, H, T] x D x D, intermediate type: fragments (bf16), row-major (fp32)
  const void* U;        // [B, H, T] x D x D tiles, intermediate type
  const float* gamma;   // [B, T, H], or nullptr for 0
  const float* z0;
  void* emit;           // [B, H, T] x D x D row-major, intermediate type
  float* zT;
  int B, H, T;
  int t0, Tc;           // frames t0 .. t0 + Tc - 1 of the T-frame tensors
  int chunk;            // 0: one walk; c > 0: chunks of c frames (see above)
  int emit_entry;       // forward: also emit the entering Z (at slot t0 - 1)
  const float* zmid;    // replay with chunk > 0: entering state of every chunk
  float* compC;         // composite output -C_w^T
  float* compH;         // composite output H_w
};
hipError_t launch_scan(const ScanArgs& a, int io, int nt, int mode, hipStream_t s);

// Token-stream product with a per-frame D x D matrix M, one wave per output
// feature tile: out[n] = M tok[n] (trans = false) or M^T tok[n] (trans =
// true).  Forward output: O_t = S_t Q^_t; backward: dQ^_t = S_t^T dO_t.
struct OutArgs {
  const void* tok;      // [B, L, H, D] io dtype (Q, or dO)
  const void* mat;      // [B, H, T] x D x D row-major, intermediate type
  void* out;            // [B, L, H, D] io dtype
  int B, H, T, N;
  int t0, Tc;           // frames t0 .. t0 + Tc - 1
  int P;                // token splits: each frame's chunks over P workgroups
  int norm;             // O_t = S_t (q / |q|) per token (forward only; 0 for a zero row)
  float* inv_out;       // with norm: 1 / |q| per row, [B, L, H] (0 for a zero row), or nullptr
};
hipError_t launch_output(const OutArgs& a, int io, int nt, bool trans, hipStream_t s);

// Backward, per (frame, head group), bf16: the two passes over dO in one,
//   X_t = dO_t Q^_t^T   (D x D per head, MFMA tile layout, bf16)
//   dQ^_t = S_t^T dO_t  (token rows, io dtype).
struct XdqArgs {
  const void* d_o;      // [B, L, H, D]
  const void* q;        // [B, L, H, D]
  const void* S;        // [B, H, T] x D x D row-major bf16: S_t
  void* X;              // [B, H, T] x D x D tiles bf16
  void* dq;             // [B, L, H, D]
  int B, H, T, N;
  // Normalised queries taken from the raw rows: q holds the raw queries and
  // inv 1 / |q| per row, [B, L, H] (0 for a zero row); the pass stages
  // q^ = q inv and dq receives the gradient of the raw rows,
  // (dq^ - q^ (q^ . dq^)) / |q|.  nullptr: q is used as given, dq = dq^.
  const float* inv;
};
// Whether launch_xdq takes a launch (bf16, 256 or more (frame, head group)
// items).
bool xdq_supported(int io, int64_t B, int64_t T, int64_t H);
// hipErrorNotSupported when the launch does not suit the fused pass (fp32,
// or fewer than 256 (frame, head group) items): the caller then runs the
// Gram-mode X pass and the transposed output pass instead.
hipError_t launch_xdq(const XdqArgs& a, int io, int nt, hipStream_t s);

// Backward, per frame: W_t = dM_t + dM_t^T with dM_t = S_{t-1}^T G_t, and
// dgamma_t = tr(dM_t).
struct DmArgs {
  const void* S;        // states after each frame, row-major, intermediate type
  const float* s0;      // [B, H, D, D] fp32 initial state or nullptr (zero)
  const void* G;        // row-major, intermediate type
  void* W;              // row-major, intermediate type
  float* dgamma;        // [B, T, H]
  int B, H, T;
};
hipError_t launch_dm(const DmArgs& a, int io, int nt, hipStream_t s);

// Backward, per frame, token pass: dK, dV, dbeta.  bf16: the pass also
// forms W_t = dM_t + dM_t^T (dM_t = S_{t-1}^T G_t) and dgamma_t = tr(dM_t)
// itself from S and G (no dm pass; W unused); fp32 reads W from dm_kernel.
struct BwdTokArgs {
  const void* k;
  const void* v;
  const float* beta;    // [B, L, H]
  const void* G;        // row-major, intermediate type
  const void* W;        // row-major, intermediate type (fp32 io)
  void* dk;
  void* dv;
  float* dbeta;         // [B, L, H]
  float s;              // key scale
  int B, H, T, N;
  const void* S;        // bf16: states after each frame, row-major
  const float* s0;      // bf16: [B, H, D, D] fp32 initial state or nullptr (zero)
  float* dgamma;        // bf16: [B, T, H]
  // bf16, normalised keys taken from the raw rows: k holds the raw keys, the
  // pass forms |k| per row from the rows it stages, uses k^ = k / |k| (0 for
  // a zero row), and dk receives the gradient of the raw rows,
  // (dk^ - k^ (k^ . dk^)) / |k|.  0: k is used as given.
  int norm;
};
hipError_t launch_bwd_tok(const BwdTokArgs& a, int io, int nt, hipStream_t s);

// Prologue of the GDN block (gdn_flag).
//   sigmoid:        y[i] = 1 / (1 + exp(-x[i])), i < n (fp32)
//   sigmoid_bwd:    g[i] <- g[i] p (1 - p), p = sigmoid(x[i])
//   rows_normalize: y[r] = x[r] / |x[r]| for rows of d io elements (0 for a
//                   zero row), unless y is nullptr; with inv, also
//                   inv[r] = 1 / |x[r]| (0 for a zero row)
//   rows_normalize_bwd: g[r] <- (g[r] - x^ (x^ . g[r])) / |x[r]| in place,
//                   x^ = x[r] / |x[r]| (0 for a zero row)
hipError_t launch_sigmoid(const float* x, float* y, int64_t n, hipStream_t s);
hipError_t launch_sigmoid_bwd(const float* x, float* g, int64_t n, hipStream_t s);
hipError_t launch_rows_normalize(const void* x, void* y, float* inv, int64_t rows, int d, int io,
                                 hipStream_t s);
hipError_t launch_rows_normalize_bwd(const void* x, void* g, int64_t rows, int d, int io,
                                     hipStream_t s);

// Direct form of the state update (short launches): per (b, h, 16-row
// block) a workgroup walks the T frames, S_t = gamma_t S_{t-1} + sum_n
// beta_n (s v_n - s^2 S_{t-1} k_n) k_n^T, straight from the token rows, and
// emits every S_t; the output kernel then forms O_t.  bf16 only.
struct DirectArgs {
  const void* k;
  const void* v;
  const float* gamma;   // [B, T, H]
  const float* beta;    // [B, L, H]
  const float* z0;      // [B, H, D, D] fp32 initial state or nullptr (zero)
  void* emit;           // [B, H, T] x D x D bf16 row-major: S_t
  float* zT;            // [B, H, D, D] fp32 final state or nullptr; may equal z0
  float s;              // key scale
  int B, H, T, N;
  float* part;          // token-split launches: [B, H, D/16, P] x D/16 x 256 fp32 partials
  int P;                // token parts (split launches)
  const void* q;        // split launches: [B, N, H, D] queries (T == 1)
  void* o;              // split launches: [B, N, H, D] outputs
};
hipError_t launch_direct(const DirectArgs& a, int nt, hipStream_t s);
// One frame (T == 1) with its tokens split over a.P parts of kDirectPartTokens:
// launch_direct_parts has every (head, part) form its part's update of every
// row block in a.part; launch_direct_out then sums them in a fixed order,
// S_1 = gamma S_0 + sum of the parts (zT), and forms the outputs o from q.
constexpr int kDirectPartTokens = 128;
hipError_t launch_direct_parts(const DirectArgs& a, int nt, hipStream_t s);
hipError_t launch_direct_out(const DirectArgs& a, int nt, hipStream_t s);

// Token-space forward (frames with few tokens): one workgroup per (b, h),
// chunks of F frames of N tokens, F N <= TokCfg<io>::CP.
template <int IO> struct TokCfg {
  static constexpr int CP = IO == IO_BF16 ? 64 : 32;   // tokens per chunk at most
};
struct TokArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;   // [B, T, H]
  const float* beta;    // [B, L, H]
  const float* z0;      // [B, H, D, D] fp32 initial state or nullptr (zero)
  void* o;              // [B, L, H, D] io dtype
  float* zT;            // [B, H, D, D] fp32 final state or nullptr; may equal z0
  float s;              // key scale
  int B, H, T, N;
  int F;                // frames per chunk
  int nck;              // chunks per sequence, ceil(T / F)
  void* ws;             // B H nck records of token_record_bytes(io) bytes
  int64_t rec_bytes;
  // Segments: nseg segments of cps chunks (the last may be shorter).
  int mode;             // TOK_PLAIN (nseg == 1), TOK_COMPOSITE, TOK_REPLAY
  int nseg, cps;
  float* compH;         // composite pass: [B, H, nseg] x D x D fp32, MFMA tile order
  float* compC;         // composite pass: -Phi^T, row-major
  const float* zin;     // replay: entering states [B, H, nseg] x D x D fp32
};
enum TokMode { TOK_PLAIN = 0, TOK_COMPOSITE = 1, TOK_REPLAY = 2 };
int64_t token_record_bytes(int io);
// prep: also run the per-chunk operator kernel first
hipError_t launch_token(const TokArgs& a, int io, int nt, bool prep, hipStream_t s);

}  // namespace gdn
