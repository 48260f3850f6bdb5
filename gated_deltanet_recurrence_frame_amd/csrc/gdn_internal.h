// Kernel argument blocks and launchers shared between the libgdn kernels and
// the host-side C ABI (gdn_api.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Token contraction C_r = scale_r X_r^T diag(w) Y per (b, t, h) frame.
struct GramArgs {
  const void* x0;      // [B, L, H, D] io dtype
  const void* x1;      // second row operand (NR == 2) or unused
  const void* y;       // column operand (NR == 1); NR == 2 uses x0
  const float* w;      // [B, L, H] per-token weights, or nullptr for 1
  float* out0;         // [B, H, T, D, D]
  float* out1;         // [B, H, T, D, D] (NR == 2)
  float scale0, scale1;
  int B, H, T, N;
};
hipError_t launch_gram(const GramArgs& a, int io, int nt, int nr, hipStream_t s);

// Inter-frame scan over the carried D x D matrix Z, 16 rows per workgroup.
//   forward  (reverse = 0), t = 0..T-1:  Z <- gamma_t Z - Z A_t + U_t; emit Z
//   backward (reverse = 1), t = T-1..0:  Z <- Z + U_t; emit Z;
//                                        Z <- gamma_t Z - Z A_t
// z0 / zT: [B, H, D, D] initial / final Z (nullptr: zero / not written).
struct ScanArgs {
  const float* A;       // [B, H, T, D, D]
  const float* U;       // [B, H, T, D, D]
  const float* gamma;   // [B, T, H]
  const float* z0;
  float* emit;          // [B, H, T, D, D] fp32
  float* zT;
  int B, H, T;
};
hipError_t launch_scan(const ScanArgs& a, int nt, bool reverse, hipStream_t s);

// Composite (chunked) forward scan: chunks of `chunk` frames.
struct ChunkScanArgs {
  const float* A;       // [B, H, T, D, D]
  const float* U;       // [B, H, T, D, D]
  const float* gamma;   // [B, T, H]
  const float* z0;      // [B, H, D, D] or nullptr
  float* emit;          // [B, H, T, D, D] states S_t
  float* zT;            // [B, H, D, D] or nullptr
  float* comp;          // [B, H, P, D, D] transition composites (workspace)
  float* hin;           // [B, H, P, D, D] input composites, then incoming states
  int B, H, T, chunk;
};
hipError_t launch_chunk_scan(const ChunkScanArgs& a, int nt, hipStream_t s);

// Token-stream products with per-frame D x D matrices, one wave per output
// feature tile.  Forward output: O_t = S_t Q^_t.
struct OutArgs {
  const void* tok;      // Q [B, L, H, D]
  const float* mat;     // S_t [B, H, T, D, D]
  void* out;            // O [B, L, H, D]
  int B, H, T, N;
};
hipError_t launch_output(const OutArgs& a, int io, int nt, hipStream_t s);

// Backward, per frame: W_t = dM_t + dM_t^T with dM_t = S_{t-1}^T G_t, and
// dgamma_t = tr(dM_t).
struct DmArgs {
  const float* S;       // [B, H, T, D, D] states after each frame
  const float* s0;      // [B, H, D, D] initial state or nullptr (zero)
  const float* G;       // [B, H, T, D, D]
  float* W;             // [B, H, T, D, D]
  float* dgamma;        // [B, T, H]
  int B, H, T;
};
hipError_t launch_dm(const DmArgs& a, int nt, hipStream_t s);

// Backward, per frame, token pass: dQ, dK, dV, dbeta.
struct BwdTokArgs {
  const void* k;
  const void* v;
  const void* d_o;
  const float* beta;    // [B, L, H]
  const float* S;       // [B, H, T, D, D] states after each frame
  const float* G;       // [B, H, T, D, D]
  const float* W;       // [B, H, T, D, D]
  void* dq;
  void* dk;
  void* dv;
  float* dbeta;         // [B, L, H]
  float s;              // key scale
  int B, H, T, N;
};
hipError_t launch_bwd_tok(const BwdTokArgs& a, int io, int nt, hipStream_t s);

}  // namespace gdn
