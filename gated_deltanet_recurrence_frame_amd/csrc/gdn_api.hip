// Host side of libgdn's C ABI: argument validation, workspace carving and
// kernel dispatch onto the caller's stream.  See include/gdn.h for the
// contract of every entry point.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

using namespace gdn;

namespace {

// Default scan: with few sequences (B H) the sequential scan leaves most
// CUs idle, and the composite prefix over chunks of frames shortens its
// chain (forward at 121 x 880 tokens, D = 112: 1 head 103 -> 83 us with
// chunks of 16, 8 heads 248 -> 230 us, 16 heads 428 -> 409 us with chunks
// of 32; 20 heads 516 vs 518 us).
int default_chunk(int64_t seqs) { return seqs <= 8 ? 16 : seqs <= 16 ? 32 : 1; }
// GDN_ALGO_AUTO takes the token form for frames of at most this many tokens
// (0: never), the direct form for bf16 launches of at most this many frames
// (streaming steps, short windows), else the frame form
constexpr int kTokenAutoMaxN = 0;
constexpr int kDirectAutoMaxT = 2;

struct Shape {
  int64_t B, H, T, N, D, L;
  int io;            // IO_BF16 / IO_F32
  int es;            // bytes per io element
  float s;           // key scale
  int chunk;         // 1: sequential scan; >= 2: composite chunks
  int64_t mat;       // bytes of one [B, H, T] x D x D buffer of the intermediate
                     // type (bf16 for bf16 io, fp32 for fp32 io)
  int64_t parts;     // composite chunks per sequence
  bool token;        // forward in token form (chunks of frames, no D x D per frame)
  bool direct;       // forward in direct form (frames in turn, from the token rows)
  int algo;          // the problem's gdn_algorithm
  bool norm;         // GDN_FLAG_NORMALIZE_QK
  bool gates;        // GDN_FLAG_GATE_LOGITS
};

gdn_status check_problem(const gdn_problem* p, Shape* sh) {
  if (!p) return GDN_ERR_NULL_POINTER;
  if (p->io_dtype != GDN_BF16 && p->io_dtype != GDN_FP32) return GDN_ERR_BAD_DTYPE;
  if (p->B < 1 || p->H < 1 || p->T < 1 || p->N < 1 || p->Dk < 1 || p->Dv < 1)
    return GDN_ERR_BAD_SHAPE;
  if (p->scan_chunk < 0) return GDN_ERR_BAD_SHAPE;
  if (!isfinite(p->key_scale)) return GDN_ERR_BAD_SHAPE;
  if (p->Dk != p->Dv || p->Dk % 16 != 0 || p->Dk > 128) return GDN_ERR_UNSUPPORTED;
  if (p->algorithm < GDN_ALGO_AUTO || p->algorithm > GDN_ALGO_DIRECT) return GDN_ERR_UNSUPPORTED;
  if (p->flags & ~(GDN_FLAG_NORMALIZE_QK | GDN_FLAG_GATE_LOGITS)) return GDN_ERR_UNSUPPORTED;
  Shape s;
  s.B = p->B; s.H = p->H; s.T = p->T; s.N = p->N; s.D = p->Dk;
  s.L = s.T * s.N;
  // Grid sizes and element offsets must fit the kernels' integer types.
  if (s.B * s.T * s.H > INT32_MAX || s.B * s.H * 8 > INT32_MAX) return GDN_ERR_BAD_SHAPE;
  if (s.B * s.L * s.H > (int64_t(1) << 40)) return GDN_ERR_BAD_SHAPE;
  s.io = p->io_dtype == GDN_BF16 ? IO_BF16 : IO_F32;
  s.es = p->io_dtype == GDN_BF16 ? 2 : 4;
  // The Gram kernel addresses a frame's token rows with 32-bit byte offsets
  // from 24-bit multiplies: one frame's rows under 2 GiB, N and a token's
  // row (H D es bytes) under 2^24.
  if (s.N >= (int64_t(1) << 24) || s.H * s.D * s.es >= (int64_t(1) << 24) ||
      s.N * s.H * s.D * s.es >= (int64_t(1) << 31))
    return GDN_ERR_BAD_SHAPE;
  s.s = p->key_scale != 0.f ? p->key_scale : (float)(1.0 / sqrt((double)s.D * (double)s.N));
  s.chunk = p->scan_chunk == 0 ? default_chunk(s.B * s.H) : p->scan_chunk;
  if (s.chunk > s.T) s.chunk = (int)s.T;
  s.mat = s.B * s.H * s.T * s.D * s.D * s.es;
  s.parts = s.chunk <= 1 ? 1 : (s.T + s.chunk - 1) / s.chunk;   // 1: sequential
  const int64_t tok_max = s.io == IO_BF16 ? TokCfg<IO_BF16>::CP : TokCfg<IO_F32>::CP;
  if (p->algorithm == GDN_ALGO_TOKEN && s.N > tok_max) return GDN_ERR_UNSUPPORTED;
  s.token = p->algorithm == GDN_ALGO_TOKEN ||
            (p->algorithm == GDN_ALGO_AUTO && s.N <= kTokenAutoMaxN);
  if (p->algorithm == GDN_ALGO_DIRECT && s.io != IO_BF16) return GDN_ERR_UNSUPPORTED;
  s.direct = p->algorithm == GDN_ALGO_DIRECT ||
             (p->algorithm == GDN_ALGO_AUTO && !s.token && s.io == IO_BF16 &&
              s.T <= kDirectAutoMaxT);
  s.algo = p->algorithm;
  s.norm = (p->flags & GDN_FLAG_NORMALIZE_QK) != 0;
  s.gates = (p->flags & GDN_FLAG_GATE_LOGITS) != 0;
  *sh = s;
  return GDN_OK;
}

// Token splits for launches with few frames (streaming steps, short
// clips): the Gram/write kernel splits a frame's token chunks over
// gram_splits workgroups (fp32 partials, then a fixed-order sum), the
// output kernel over out_splits workgroups.
int gram_splits(const Shape& s) {
  // the Gram kernel takes adjacent head pairs when H is even
  const int64_t hpw = s.H % 2 == 0 ? 2 : 1;
  const int64_t wgs = s.B * s.T * (s.H / hpw);     // workgroups without splits
  if (wgs >= 256) return 1;
  const int64_t ct = s.io == IO_BF16 ? 32 : 16;     // the Gram kernel's token chunk
  int64_t p = (256 + wgs - 1) / wgs;
  const int64_t nch = (s.N + ct - 1) / ct;
  if (p > nch) p = nch;
  if (p > 8) p = 8;
  return (int)(p < 1 ? 1 : p);
}
int out_splits(const Shape& s) {
  // the output kernel takes adjacent head pairs when H is even
  const int64_t hpw = s.H % 2 == 0 ? 2 : 1;
  const int64_t frames = s.B * s.T * (s.H / hpw);
  if (frames >= 512) return 1;
  const int64_t ct = (s.io == IO_BF16 ? 64 : 32) / hpw;
  int64_t p = (512 + frames - 1) / frames;
  const int64_t nch = (s.N + ct - 1) / ct;
  if (p > nch) p = nch;
  return (int)(p < 1 ? 1 : p);
}
int64_t partial_bytes(const Shape& s, int nr) {
  const int p = gram_splits(s);
  return p > 1 ? (int64_t)p * s.B * s.H * s.T * nr * s.D * s.D * 4 : 0;
}

// Chunked scan: -C_w^T, H_w and the entering state of every chunk, fp32.
int64_t composite_bytes(const Shape& s) {
  return s.parts > 1 ? 3 * s.B * s.H * s.parts * s.D * s.D * 4 : 0;
}
// One-frame launches in direct form split the frame's tokens into parts
// (when it has more than one part's worth) and keep every part's update of
// the state in fp32.  At most kMaxDirectParts parts (frames of up to 4096
// tokens): the parts' workspace grows with the frame, and longer frames walk
// their chunks in one workgroup as for several frames.  The parts' grid
// stays within int32.
constexpr int64_t kMaxDirectParts = 32;
int64_t direct_parts(const Shape& s) {
  if (!s.direct || s.T != 1) return 0;
  const int64_t p = (s.N + kDirectPartTokens - 1) / kDirectPartTokens;
  if (p < 2 || p > kMaxDirectParts || s.B * s.H * (s.D / 16) * p > INT32_MAX) return 0;
  return p;
}
int64_t direct_part_bytes(const Shape& s) { return direct_parts(s) * s.B * s.H * s.D * s.D * 4; }
// The token-split partials (used by the Gram launches), the composites
// (used by the scans) and the direct form's parts are never live at the
// same time on the stream, so they share one region after the D x D
// buffers.
int64_t scratch_bytes(const Shape& s) {
  const int64_t a = partial_bytes(s, 2), b = composite_bytes(s), c = direct_part_bytes(s);
  const int64_t m = a > b ? a : b;
  return m > c ? m : c;
}

}  // namespace

// Bytes of one chunk's operator record of the token form (two CP x CP
// token matrices in the io type, five fp32 vectors of CP).
int64_t gdn::token_record_bytes(int io) {
  const int cp = io == IO_BF16 ? TokCfg<IO_BF16>::CP : TokCfg<IO_F32>::CP;
  const int es = io == IO_BF16 ? 2 : 4;
  return (int64_t)2 * cp * cp * es + 5 * cp * 4;
}

namespace {

// Token form: per-chunk operators of F = CP / N frames for every (b, h).
int64_t token_frames(const Shape& s) {
  return (s.io == IO_BF16 ? TokCfg<IO_BF16>::CP : TokCfg<IO_F32>::CP) / s.N;
}
int64_t token_chunks(const Shape& s) {
  const int64_t F = token_frames(s);
  return (s.T + F - 1) / F;
}
// Segments walked in parallel: about 256 (b, h, segment) items (two walks
// each in the composite pass), at least 8 chunks per segment.  (Token-wise
// GDN at 106,480 tokens and 20 heads, before the prep kernel staged its
// rows: 4.17 ms with 128 items, 3.52 with 256, 3.55 with 512.)
int64_t token_segments(const Shape& s) {
  int64_t n = 256 / (s.B * s.H);
  const int64_t most = token_chunks(s) / 8;
  if (n > most) n = most;
  return n < 1 ? 1 : n;
}
int64_t token_ws(const Shape& s) {
  const int64_t seg = token_segments(s);
  const int64_t comp = seg > 1 ? 3 * s.B * s.H * seg * s.D * s.D * 4 : 0;
  return s.B * s.H * token_chunks(s) * token_record_bytes(s.io) + comp;
}
// Prologue (gdn_flag) buffers, after everything else in the workspace:
// the gates from logits (gamma [B, T, H], beta [B, L, H], fp32) and, where
// the kernels take normalised rows as input (`copies`: the token form, the
// backward), q / |q| and k / |k| as [B, L, H, D] io dtype.
int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }
struct Prologue {
  int64_t gamma, beta, q, k, iq, end;   // offsets from the region's start; end = bytes
};
// `fused`: the backward's token passes normalise the raw rows themselves
// and take dq, dk through the chain rule; only 1 / |q| per row is kept
// (no copies)
Prologue prologue_layout(const Shape& s, bool copies, bool fused = false) {
  Prologue r{};
  int64_t o = 0;
  if (s.gates) {
    r.gamma = o; o += round256(s.B * s.T * s.H * 4);
    r.beta = o;  o += round256(s.B * s.L * s.H * 4);
  }
  if (s.norm && fused) {
    r.iq = o; o += round256(s.B * s.L * s.H * 4);
  } else if (s.norm && copies) {
    const int64_t tok = round256(s.B * s.L * s.H * s.D * s.es);
    r.q = o; o += tok;
    r.k = o; o += tok;
  }
  r.end = o;
  return r;
}
// (the region starts 256-aligned after the entry point's own buffers)
int64_t forward_base(const Shape& s) {
  return round256(s.token ? token_ws(s) : 3 * s.mat + scratch_bytes(s));
}
int64_t backward_base(const Shape& s) { return round256(6 * s.mat + scratch_bytes(s)); }
// The saved buffer: A_t, S_t, then with normalised rows 1 / |q| per row
// (fp32 [B, L, H]), which the output pass computes anyway.
int64_t saved_bytes(const Shape& s) { return 2 * s.mat + (s.norm ? s.B * s.L * s.H * 4 : 0); }
// The direct form takes normalised copies of q and k too; it falls back to
// the frame form (same workspace start) when a saved buffer is asked for.
bool forward_copies(const Shape& s) { return s.token || s.direct; }
int64_t forward_ws(const Shape& s) {
  const int64_t pro = prologue_layout(s, forward_copies(s)).end;
  return pro ? forward_base(s) + pro : (s.token ? token_ws(s) : 3 * s.mat + scratch_bytes(s));
}
// With normalised rows the bf16 backward's token passes (the one-pass dO
// kernel and the dK/dV pass) take the raw q and k, normalise them as they
// stage them and apply the chain rule to dq and dk themselves; otherwise
// (fp32, launches too short for the one-pass dO kernel) the backward runs
// on normalised copies and the chain rule runs in passes of its own.
bool backward_fused_norm(const Shape& s) {
  return s.norm && xdq_supported(s.io, s.B, s.T, s.H);
}
int64_t backward_ws(const Shape& s) {
  const int64_t pro = prologue_layout(s, true, backward_fused_norm(s)).end;
  return pro ? backward_base(s) + pro : 6 * s.mat + scratch_bytes(s);
}

// Inputs of the recurrence after the prologue: the caller's tensors, or
// the workspace copies the prologue's kernels write (gates from logits;
// normalised rows when `copies`).
struct Inputs {
  const void* q;
  const void* k;
  const float* gamma;
  const float* beta;
  const float* inv_q;   // fused: 1 / |q| per row (q, k raw), else nullptr
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

struct Span {
  const void* p;
  int64_t n;
};
bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n <= 0 || b.n <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + (uintptr_t)b.n && b0 < a0 + (uintptr_t)a.n;
}
bool any_overlap(const Span* outs, int no, const Span* ins, int ni) {
  for (int i = 0; i < no; ++i)
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i], ins[j])) return true;
  for (int i = 0; i < no; ++i)
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return true;
  return false;
}

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

gdn_status run_prologue(const Shape& s, bool copies, const void* q, const void* k,
                        const float* gamma, const float* beta, char* region, Inputs* in,
                        hipStream_t stream, bool fused = false,
                        const float* given_inv_q = nullptr) {
  const Prologue pl = prologue_layout(s, copies, fused);
  *in = Inputs{q, k, gamma, beta, nullptr};
  hipError_t e = hipSuccess;
  if (s.gates) {
    float* g = reinterpret_cast<float*>(region + pl.gamma);
    float* b = reinterpret_cast<float*>(region + pl.beta);
    e = launch_sigmoid(gamma, g, s.B * s.T * s.H, stream);
    if (e == hipSuccess) e = launch_sigmoid(beta, b, s.B * s.L * s.H, stream);
    in->gamma = g;
    in->beta = b;
  }
  const int64_t rows = s.B * s.L * s.H;
  if (e == hipSuccess && s.norm && fused) {
    // 1 / |q| per row only (from the saved buffer when the forward kept
    // it); q and k stay raw
    if (given_inv_q) {
      in->inv_q = given_inv_q;
    } else {
      float* iq = reinterpret_cast<float*>(region + pl.iq);
      e = launch_rows_normalize(q, nullptr, iq, rows, (int)s.D, s.io, stream);
      in->inv_q = iq;
    }
  } else if (e == hipSuccess && s.norm && copies) {
    void* qn = region + pl.q;
    void* kn = region + pl.k;
    e = launch_rows_normalize(q, qn, nullptr, rows, (int)s.D, s.io, stream);
    if (e == hipSuccess) e = launch_rows_normalize(k, kn, nullptr, rows, (int)s.D, s.io, stream);
    in->q = qn;
    in->k = kn;
  }
  return hip_status(e);
}

// Inter-frame scan over the whole sequence, sequential or chunked
// (composites, a fold over chunks, then a parallel replay of every chunk).
gdn_status run_scan(const Shape& s, const void* A, const void* U, const float* gamma,
                    const float* z0, void* emit, float* zT, bool reverse, char* scratch,
                    hipStream_t stream) {
  const int nt = (int)(s.D / 16);
  ScanArgs sa{};
  sa.A = A; sa.U = U; sa.gamma = gamma; sa.z0 = z0; sa.emit = emit; sa.zT = zT;
  sa.B = (int)s.B; sa.H = (int)s.H; sa.T = (int)s.T;
  sa.t0 = 0; sa.Tc = (int)s.T;
  const int mode = reverse ? SCAN_REV : SCAN_FWD;
  if (s.parts <= 1) return hip_status(launch_scan(sa, s.io, nt, mode, stream));

  const int64_t cm = s.B * s.H * s.parts * s.D * s.D;   // floats per composite buffer
  float* compC = reinterpret_cast<float*>(scratch);
  float* compH = compC + cm;
  float* zmid = compH + cm;
  ScanArgs ca = sa;
  ca.z0 = nullptr; ca.emit = nullptr; ca.zT = nullptr;
  ca.chunk = s.chunk; ca.compC = compC; ca.compH = compH;
  gdn_status st = hip_status(
      launch_scan(ca, s.io, nt, reverse ? SCAN_COMP_REV : SCAN_COMP_FWD, stream));
  if (st != GDN_OK) return st;

  // Fold: Z_{w+1} = Z_w C_w + H_w, in fp32, emitting every chunk's entering state.
  ScanArgs fa{};
  fa.A = compC; fa.U = compH; fa.gamma = nullptr; fa.z0 = z0;
  fa.emit = zmid + s.D * s.D;   // slot t + 1 receives the state after chunk t
  fa.emit_entry = 1;            // slot 0 receives z0 itself
  fa.B = (int)s.B; fa.H = (int)s.H; fa.T = (int)s.parts;
  fa.t0 = 0; fa.Tc = (int)s.parts - 1;
  st = hip_status(launch_scan(fa, IO_F32, nt, SCAN_FWD, stream));
  if (st != GDN_OK) return st;

  sa.chunk = s.chunk; sa.zmid = zmid;
  return hip_status(launch_scan(sa, s.io, nt, mode, stream));
}

gdn_status record(void* const* events, int i, hipStream_t stream) {
  if (!events) return GDN_OK;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(events[i]), stream));
}

// Token-form forward: the per-chunk operators into the workspace, then the
// state pass.  The phase events of gdn_forward_events bracket both as the
// output phase (the caller records the first three).
gdn_status run_token(const Shape& s, const void* q, const void* k, const void* v,
                     const float* gamma, const float* beta, const float* state_in, void* o,
                     float* state_out, void* workspace, hipStream_t stream,
                     void* const* events) {
  TokArgs ta{};
  ta.q = q; ta.k = k; ta.v = v; ta.gamma = gamma; ta.beta = beta;
  ta.z0 = state_in; ta.o = o; ta.zT = state_out; ta.s = s.s;
  ta.B = (int)s.B; ta.H = (int)s.H; ta.T = (int)s.T; ta.N = (int)s.N;
  ta.F = (int)token_frames(s);
  ta.nck = (int)token_chunks(s);
  ta.ws = workspace;
  ta.rec_bytes = token_record_bytes(s.io);
  const int nt = (int)(s.D / 16);
  const int nseg = (int)token_segments(s);
  ta.nseg = nseg;
  ta.cps = (ta.nck + nseg - 1) / nseg;
  ta.nseg = (ta.nck + ta.cps - 1) / ta.cps;   // no empty segment
  gdn_status st = GDN_OK;
  if (ta.nseg == 1) {
    ta.mode = TOK_PLAIN;
    st = hip_status(launch_token(ta, s.io, nt, true, stream));
    if (st != GDN_OK) return st;
    return record(events, 3, stream);
  }
  // composites of every segment, the fold, then the replay of every segment
  const int64_t cm = s.B * s.H * ta.nseg * s.D * s.D;   // floats per buffer
  float* comp = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         s.B * s.H * ta.nck * ta.rec_bytes);
  ta.compH = comp;
  ta.compC = comp + cm;
  float* zmid = comp + 2 * cm;
  ta.mode = TOK_COMPOSITE;
  st = hip_status(launch_token(ta, s.io, nt, true, stream));
  if (st != GDN_OK) return st;
  ScanArgs fa{};
  fa.A = ta.compC; fa.U = ta.compH; fa.gamma = nullptr; fa.z0 = state_in;
  fa.emit = zmid + s.D * s.D;   // slot p + 1 receives the state after segment p
  fa.emit_entry = 1;            // slot 0 receives z0 itself
  fa.B = (int)s.B; fa.H = (int)s.H; fa.T = ta.nseg;
  fa.t0 = 0; fa.Tc = ta.nseg - 1;
  st = hip_status(launch_scan(fa, IO_F32, nt, SCAN_FWD, stream));
  if (st != GDN_OK) return st;
  ta.mode = TOK_REPLAY;
  ta.zin = zmid;
  st = hip_status(launch_token(ta, s.io, nt, false, stream));
  if (st != GDN_OK) return st;
  return record(events, 3, stream);
}


// Forward pipeline shared by gdn_forward and gdn_step.

gdn_status run_forward(const Shape& s, const void* q, const void* k, const void* v,
                       const float* gamma, const float* beta, const float* state_in,
                       void* o, float* state_out, void* saved, void* workspace,
                       hipStream_t stream, void* const* events = nullptr) {
  char* ws = static_cast<char*>(workspace);
  // phases: the token form's prologue and passes all count as the output
  // phase; the frame and direct forms' prologue as part of the Gram/write
  // phase, the direct form's update as the scan phase
  gdn_status st = GDN_OK;
  for (int i = 0; i < (s.token ? 3 : 1) && st == GDN_OK; ++i) st = record(events, i, stream);
  if (st != GDN_OK) return st;
  // the prologue's gates (and, for the token and direct forms, normalised rows)
  const bool direct = s.direct && !saved;
  Inputs in;
  st = run_prologue(s, s.token || direct, q, k, gamma, beta, ws + forward_base(s), &in, stream);
  if (st != GDN_OK) return st;
  q = in.q; k = in.k; gamma = in.gamma; beta = in.beta;
  if (s.token)
    return run_token(s, q, k, v, gamma, beta, state_in, o, state_out, workspace, stream, events);
  if (direct) {
    // the state update in direct form (the scan phase), then the outputs
    // from the emitted states
    void* S = ws + s.mat;
    DirectArgs da{};
    da.k = k; da.v = v; da.gamma = gamma; da.beta = beta;
    da.z0 = state_in; da.emit = S; da.zT = state_out; da.s = s.s;
    da.B = (int)s.B; da.H = (int)s.H; da.T = (int)s.T; da.N = (int)s.N;
    st = record(events, 1, stream);
    if (st != GDN_OK) return st;
    if (direct_parts(s) >= 2) {
      // one frame of many tokens: every part's update, then their sum with
      // the outputs of each row block's features
      da.part = reinterpret_cast<float*>(ws + 3 * s.mat);
      da.P = (int)direct_parts(s);
      da.q = q; da.o = o;
      st = hip_status(launch_direct_parts(da, (int)(s.D / 16), stream));
      if (st != GDN_OK) return st;
      st = record(events, 2, stream);
      if (st != GDN_OK) return st;
      st = hip_status(launch_direct_out(da, (int)(s.D / 16), stream));
      if (st != GDN_OK) return st;
      return record(events, 3, stream);
    }
    st = hip_status(launch_direct(da, (int)(s.D / 16), stream));
    if (st != GDN_OK) return st;
    st = record(events, 2, stream);
    if (st != GDN_OK) return st;
    OutArgs oa{};
    oa.tok = q; oa.mat = S; oa.out = o;
    oa.B = (int)s.B; oa.H = (int)s.H; oa.T = (int)s.T; oa.N = (int)s.N;
    oa.t0 = 0; oa.Tc = (int)s.T;
    oa.P = out_splits(s);
    st = hip_status(launch_output(oa, s.io, (int)(s.D / 16), false, stream));
    if (st != GDN_OK) return st;
    return record(events, 3, stream);
  }
  void* A = saved ? saved : ws;
  void* S = saved ? static_cast<char*>(saved) + s.mat : ws + s.mat;
  void* U = ws + 2 * s.mat;
  const int nt = (int)(s.D / 16);

  GramArgs ga{};
  ga.x0 = k; ga.x1 = v; ga.y = k; ga.w = beta;
  ga.out0 = A; ga.out1 = U;
  ga.layout0 = s.io == IO_BF16 ? LAYOUT_FRAG : LAYOUT_ROWMAJOR; ga.layout1 = LAYOUT_TILES;
  ga.scale0 = s.s * s.s; ga.scale1 = s.s;
  ga.B = (int)s.B; ga.H = (int)s.H; ga.T = (int)s.T; ga.N = (int)s.N;
  ga.t0 = 0; ga.Tc = (int)s.T;
  ga.P = gram_splits(s);
  ga.part = reinterpret_cast<float*>(ws + 3 * s.mat);
  ga.norm = s.norm;   // fused: norms of the staged key rows
  st = hip_status(launch_gram(ga, s.io, nt, 2, stream));
  if (st != GDN_OK) return st;
  if (ga.P > 1 && (st = hip_status(launch_gram_reduce(ga, s.io, nt, 2, stream))) != GDN_OK)
    return st;
  st = record(events, 1, stream);
  if (st != GDN_OK) return st;

  st = run_scan(s, A, U, gamma, state_in, S, state_out, false, ws + 3 * s.mat, stream);
  if (st != GDN_OK) return st;
  st = record(events, 2, stream);
  if (st != GDN_OK) return st;

  OutArgs oa{};
  oa.tok = q; oa.mat = S; oa.out = o;
  oa.B = (int)s.B; oa.H = (int)s.H; oa.T = (int)s.T; oa.N = (int)s.N;
  oa.t0 = 0; oa.Tc = (int)s.T;
  oa.P = out_splits(s);
  oa.norm = s.norm;   // fused: norms of the staged query rows
  if (saved && s.norm) oa.inv_out = reinterpret_cast<float*>(static_cast<char*>(saved) + 2 * s.mat);
  st = hip_status(launch_output(oa, s.io, nt, false, stream));
  if (st != GDN_OK) return st;
  return record(events, 3, stream);
}

// Static scratch of gdn_forward_noalloc: the forward's workspace for callers
// that cannot allocate.  One copy per GPU, held until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address of each GPU's copy is taken once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch (nullptr on failure).
void* device_scratch(int dev) {
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "bad shape or size";
    case GDN_ERR_BAD_DTYPE: return "unknown io dtype";
    case GDN_ERR_MISALIGNED: return "a pointer is misaligned (16 bytes; 4 for gates)";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GDN_ERR_UNSUPPORTED:
      return "unsupported: head dims (need Dk == Dv, a multiple of 16, <= 128), algorithm, "
             "or the token form's limits (N <= 64 bf16 / 32 fp32, no saved buffer)";
    case GDN_ERR_HIP: return "HIP kernel launch failed";
    case GDN_ERR_ALIASING: return "an output overlaps an input";
    case GDN_ERR_SCRATCH_TOO_SMALL:
      return "the problem needs more workspace than the static scratch of gdn_forward_noalloc "
             "holds (GDN_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

gdn_status gdn_workspace_size(const gdn_problem* p, int op, size_t* bytes) {
  if (!bytes) return GDN_ERR_NULL_POINTER;
  Shape s;
  gdn_status st = check_problem(p, &s);
  if (st != GDN_OK) return st;
  switch (op) {
    case GDN_OP_FORWARD: *bytes = (size_t)forward_ws(s); return GDN_OK;
    case GDN_OP_STEP:
      if (s.T != 1) return GDN_ERR_BAD_SHAPE;
      *bytes = (size_t)forward_ws(s);
      return GDN_OK;
    case GDN_OP_BACKWARD: *bytes = (size_t)backward_ws(s); return GDN_OK;
  }
  return GDN_ERR_BAD_SHAPE;
}

gdn_status gdn_saved_size(const gdn_problem* p, size_t* bytes) {
  if (!bytes) return GDN_ERR_NULL_POINTER;
  Shape s;
  gdn_status st = check_problem(p, &s);
  if (st != GDN_OK) return st;
  // the token and direct forms keep no A_t, S_t (GDN_ALGO_AUTO's direct
  // form gives way to the frame form when a saved buffer is passed)
  if (s.token || s.algo == GDN_ALGO_DIRECT) return GDN_ERR_UNSUPPORTED;
  *bytes = (size_t)saved_bytes(s);
  return GDN_OK;
}

static gdn_status forward_checked(const gdn_problem* p, const void* q, const void* k,
                                  const void* v, const float* gamma, const float* beta,
                                  const float* state_in, void* o, float* state_out, void* saved,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* const* events) {
  Shape s;
  gdn_status st = check_problem(p, &s);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !gamma || !beta || !o || !workspace) return GDN_ERR_NULL_POINTER;
  const void* ptrs[] = {q, k, v, state_in, o, state_out, saved, workspace};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return GDN_ERR_MISALIGNED;
  if (!aligned4(gamma) || !aligned4(beta)) return GDN_ERR_MISALIGNED;
  if ((int64_t)workspace_bytes < forward_ws(s)) return GDN_ERR_WORKSPACE_TOO_SMALL;
  if ((s.token || s.algo == GDN_ALGO_DIRECT) && saved)
    return GDN_ERR_UNSUPPORTED;   // no per-frame intermediates
  const int64_t tok = s.B * s.L * s.H * s.D * s.es;
  const int64_t stb = s.B * s.H * s.D * s.D * 4;
  const Span ins[] = {{q, tok}, {k, tok}, {v, tok}, {gamma, s.B * s.T * s.H * 4},
                      {beta, s.B * s.L * s.H * 4}, {state_in, stb}};
  const Span outs[] = {{o, tok}, {saved, saved ? saved_bytes(s) : 0},
                       {workspace, (int64_t)workspace_bytes}};
  if (any_overlap(outs, 3, ins, 6)) return GDN_ERR_ALIASING;
  if (state_out) {
    const Span so[] = {{state_out, stb}};
    if (any_overlap(so, 1, outs, 3)) return GDN_ERR_ALIASING;
    if (state_out != state_in && any_overlap(so, 1, ins, 6)) return GDN_ERR_ALIASING;
  }
  return run_forward(s, q, k, v, gamma, beta, state_in, o, state_out, saved, workspace,
                     static_cast<hipStream_t>(stream), events);
}

gdn_status gdn_forward(const gdn_problem* p, const void* q, const void* k, const void* v,
                       const float* gamma, const float* beta, const float* state_in,
                       void* o, float* state_out, void* saved, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return forward_checked(p, q, k, v, gamma, beta, state_in, o, state_out, saved, workspace,
                         workspace_bytes, stream, nullptr);
}

gdn_status gdn_forward_events(const gdn_problem* p, const void* q, const void* k,
                              const void* v, const float* gamma, const float* beta,
                              const float* state_in, void* o, float* state_out, void* saved,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void* const* events) {
  if (!events) return GDN_ERR_NULL_POINTER;
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return GDN_ERR_NULL_POINTER;
  return forward_checked(p, q, k, v, gamma, beta, state_in, o, state_out, saved, workspace,
                         workspace_bytes, stream, events);
}

gdn_status gdn_forward_noalloc(const gdn_problem* p, const void* q, const void* k,
                               const void* v, const float* gamma, const float* beta,
                               const float* state_in, void* o, float* state_out, void* saved,
                               void* stream) {
  Shape s;
  gdn_status st = check_problem(p, &s);
  if (st != GDN_OK) return st;
  const int64_t need = forward_ws(s);
  if (need > (int64_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH_TOO_SMALL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
  void* ws = device_scratch(dev);
  if (!ws) return GDN_ERR_HIP;
  // nothing in the forward's workspace needs to start at zero: every
  // intermediate is written before it is read within the call
  return forward_checked(p, q, k, v, gamma, beta, state_in, o, state_out, saved, ws,
                         (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

gdn_status gdn_step(const gdn_problem* p, const void* q, const void* k, const void* v,
                    const float* gamma, const float* beta, float* state, void* o,
                    void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  gdn_status st = check_problem(p, &s);
  if (st != GDN_OK) return st;
  if (s.T != 1) return GDN_ERR_BAD_SHAPE;
  if (!state) return GDN_ERR_NULL_POINTER;
  return gdn_forward(p, q, k, v, gamma, beta, state, o, state, nullptr, workspace,
                     workspace_bytes, stream);
}

gdn_status gdn_backward(const gdn_problem* p, const void* q, const void* k, const void* v,
                        const float* gamma, const float* beta, const float* state_in,
                        const void* d_o, const float* d_state_out, const void* saved,
                        void* dq, void* dk, void* dv, float* dgamma, float* dbeta,
                        float* d_state_in, void* workspace, size_t workspace_bytes,
                        void* stream) {
  Shape s;
  gdn_status st = check_problem(p, &s);
  if (st != GDN_OK) return st;
  if (!q || !k || !v || !gamma || !beta || !d_o || !dq || !dk || !dv || !dgamma || !dbeta ||
      !workspace)
    return GDN_ERR_NULL_POINTER;
  const void* ptrs[] = {q, k, v, state_in, d_o, d_state_out, saved,
                        dq, dk, dv, d_state_in, workspace};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return GDN_ERR_MISALIGNED;
  const void* gates[] = {gamma, beta, dgamma, dbeta};
  for (const void* x : gates)
    if (!aligned4(x)) return GDN_ERR_MISALIGNED;
  if ((int64_t)workspace_bytes < backward_ws(s)) return GDN_ERR_WORKSPACE_TOO_SMALL;
  const int64_t tok = s.B * s.L * s.H * s.D * s.es;
  const int64_t stb = s.B * s.H * s.D * s.D * 4;
  const Span ins[] = {{q, tok}, {k, tok}, {v, tok}, {gamma, s.B * s.T * s.H * 4},
                      {beta, s.B * s.L * s.H * 4}, {state_in, stb}, {d_o, tok},
                      {d_state_out, stb}, {saved, saved ? saved_bytes(s) : 0}};
  const Span outs[] = {{dq, tok}, {dk, tok}, {dv, tok}, {dgamma, s.B * s.T * s.H * 4},
                       {dbeta, s.B * s.L * s.H * 4}, {d_state_in, stb},
                       {workspace, (int64_t)workspace_bytes}};
  if (any_overlap(outs, 7, ins, 9)) return GDN_ERR_ALIASING;

  hipStream_t stream_ = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int nt = (int)(s.D / 16);
  // The prologue's outputs (normalised q, k and the gates, in the
  // workspace) are the inputs of the recurrence's reverse pass; its chain
  // rule runs at the end on dq, dk, dgamma, dbeta in place.
  const void* q_raw = q;
  const void* k_raw = k;
  const float* gamma_raw = gamma;
  const float* beta_raw = beta;
  Inputs in;
  const bool fused = backward_fused_norm(s);
  const float* saved_inv_q =
      saved && s.norm ? reinterpret_cast<const float*>(static_cast<const char*>(saved) + 2 * s.mat)
                      : nullptr;
  st = run_prologue(s, true, q, k, gamma, beta, ws + backward_base(s), &in, stream_, fused,
                    saved_inv_q);
  if (st != GDN_OK) return st;
  q = in.q; k = in.k; gamma = in.gamma; beta = in.beta;
  const void* A;
  const void* S;
  if (saved) {
    A = saved;
    S = static_cast<const char*>(saved) + s.mat;
  } else {
    // Recompute A_t and S_t with the forward's own kernels into the
    // workspace (layout of `saved`), without writing an output.
    void* A_ = ws;
    void* S_ = ws + s.mat;
    void* U_ = ws + 2 * s.mat;
    GramArgs ga{};
    ga.x0 = k; ga.x1 = v; ga.y = k; ga.w = beta; ga.out0 = A_; ga.out1 = U_;
    ga.layout0 = s.io == IO_BF16 ? LAYOUT_FRAG : LAYOUT_ROWMAJOR; ga.layout1 = LAYOUT_TILES;
    ga.scale0 = s.s * s.s; ga.scale1 = s.s;
    ga.B = (int)s.B; ga.H = (int)s.H; ga.T = (int)s.T; ga.N = (int)s.N;
    ga.t0 = 0; ga.Tc = (int)s.T;
    ga.P = gram_splits(s);
    ga.part = reinterpret_cast<float*>(ws + 6 * s.mat);
    ga.norm = fused;   // raw keys: norms of the staged rows, as in the forward
    st = hip_status(launch_gram(ga, s.io, nt, 2, stream_));
    if (st != GDN_OK) return st;
    if (ga.P > 1 && (st = hip_status(launch_gram_reduce(ga, s.io, nt, 2, stream_))) != GDN_OK)
      return st;
    st = run_scan(s, A_, U_, gamma, state_in, S_, nullptr, false, ws + 6 * s.mat, stream_);
    if (st != GDN_OK) return st;
    A = A_;
    S = S_;
  }
  void* X = ws + 3 * s.mat;
  void* G = ws + 4 * s.mat;
  void* W = ws + 5 * s.mat;

  // X_t = dO_t Q^_t^T, the frame's own contribution to dLoss/dS_t, and
  // dQ^_t = S_t^T dO_t: one pass over dO where it suits (bf16, enough
  // frames), else a Gram-mode pass for X_t here and the transposed output
  // pass for dQ below.
  XdqArgs xa{};
  xa.d_o = d_o; xa.q = q; xa.S = S; xa.X = ws + 3 * s.mat; xa.dq = dq;
  xa.B = (int)s.B; xa.H = (int)s.H; xa.T = (int)s.T; xa.N = (int)s.N;
  xa.inv = in.inv_q;   // fused: raw queries, dq of the raw rows
  hipError_t xe = launch_xdq(xa, s.io, nt, stream_);
  if (xe != hipSuccess && (xe != hipErrorNotSupported || fused)) return GDN_ERR_HIP;
  const bool fused_dq = xe == hipSuccess;
  GramArgs gx{};
  gx.x0 = d_o; gx.x1 = nullptr; gx.y = q; gx.w = nullptr; gx.out0 = X; gx.out1 = nullptr;
  gx.layout0 = LAYOUT_TILES; gx.layout1 = LAYOUT_TILES;
  gx.scale0 = 1.f; gx.scale1 = 0.f;
  gx.B = (int)s.B; gx.H = (int)s.H; gx.T = (int)s.T; gx.N = (int)s.N;
  gx.t0 = 0; gx.Tc = (int)s.T;
  gx.P = gram_splits(s);
  gx.part = reinterpret_cast<float*>(ws + 6 * s.mat);
  if (!fused_dq) {
    st = hip_status(launch_gram(gx, s.io, nt, 1, stream_));
    if (st != GDN_OK) return st;
    if (gx.P > 1 && (st = hip_status(launch_gram_reduce(gx, s.io, nt, 1, stream_))) != GDN_OK)
      return st;
  }

  // Reverse scan: G_t = X_t + G_{t+1} M_{t+1}^T, dS_0 = G_1 M_1^T.
  st = run_scan(s, A, X, gamma, d_state_out, G, d_state_in, true, ws + 6 * s.mat, stream_);
  if (st != GDN_OK) return st;

  // W_t = dM_t + dM_t^T and dgamma_t: a pass of their own for fp32; the
  // bf16 dK/dV pass forms them from S and G itself
  if (s.io != IO_BF16) {
    DmArgs da{};
    da.S = S; da.s0 = state_in; da.G = G; da.W = W; da.dgamma = dgamma;
    da.B = (int)s.B; da.H = (int)s.H; da.T = (int)s.T;
    st = hip_status(launch_dm(da, s.io, nt, stream_));
    if (st != GDN_OK) return st;
  }

  if (!fused_dq) {
    // dQ^_t = S_t^T dO_t: the output kernel on the transposed states.
    OutArgs qa{};
    qa.tok = d_o; qa.mat = S; qa.out = dq;
    qa.B = (int)s.B; qa.H = (int)s.H; qa.T = (int)s.T; qa.N = (int)s.N;
    qa.t0 = 0; qa.Tc = (int)s.T;
    qa.P = out_splits(s);
    st = hip_status(launch_output(qa, s.io, nt, true, stream_));
    if (st != GDN_OK) return st;
  }

  BwdTokArgs ba{};
  ba.k = k; ba.v = v; ba.beta = beta; ba.G = G; ba.W = W;
  ba.dk = dk; ba.dv = dv; ba.dbeta = dbeta; ba.s = s.s;
  ba.B = (int)s.B; ba.H = (int)s.H; ba.T = (int)s.T; ba.N = (int)s.N;
  ba.S = S; ba.s0 = state_in; ba.dgamma = dgamma;
  ba.norm = fused;   // raw keys normalised in the pass, dk of the raw rows
  st = hip_status(launch_bwd_tok(ba, s.io, nt, stream_));
  if (st != GDN_OK) return st;

  // Chain rule through the prologue (what the token passes did not take).
  hipError_t e = hipSuccess;
  if (s.norm) {
    const int64_t rows = s.B * s.L * s.H;
    if (!fused) {
      e = launch_rows_normalize_bwd(q_raw, dq, rows, (int)s.D, s.io, stream_);
      if (e == hipSuccess) e = launch_rows_normalize_bwd(k_raw, dk, rows, (int)s.D, s.io, stream_);
    }
  }
  if (e == hipSuccess && s.gates) {
    e = launch_sigmoid_bwd(gamma_raw, dgamma, s.B * s.T * s.H, stream_);
    if (e == hipSuccess) e = launch_sigmoid_bwd(beta_raw, dbeta, s.B * s.L * s.H, stream_);
  }
  return hip_status(e);
}

}  // extern "C"
