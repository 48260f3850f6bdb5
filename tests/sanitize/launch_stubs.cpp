// Host-only stand-ins for libgdn's kernel launchers, for the sanitizer build
// of the C ABI's host code (gdn_api.hip): nothing is launched.  Every
// launcher records its call and checks that each device pointer it receives
// lies inside one of the regions api_driver.cpp handed to the entry point (the
// caller's tensors and workspace), together with the extent the launch would
// touch where that follows from its arguments.  Violations are counted and
// reported by api_driver.cpp.
#include <stdint.h>
#include <stdio.h>

#include "gdn_internal.h"
#include "sanitize_regions.h"

namespace {

struct Region {
  uintptr_t base;
  int64_t bytes;
};
Region g_regions[64];
int g_nregions = 0;
int g_calls = 0;
int g_bad = 0;

// [p, p + bytes) inside one registered region (a null pointer is not checked)
void need(const void* p, int64_t bytes, const char* what) {
  if (!p) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  for (int i = 0; i < g_nregions; ++i) {
    const Region& r = g_regions[i];
    if (a >= r.base && bytes >= 0 && a + (uintptr_t)bytes <= r.base + (uintptr_t)r.bytes) return;
  }
  ++g_bad;
  fprintf(stderr, "launch stub: %s at %p (+%lld bytes) outside every region\n", what, p,
          (long long)bytes);
}

int64_t es_of(int io) { return io == gdn::IO_BF16 ? 2 : 4; }

}  // namespace

extern "C" void sanitize_reset(void) {
  g_nregions = 0;
  g_calls = 0;
  g_bad = 0;
}
extern "C" void sanitize_region(const void* base, int64_t bytes) {
  if (base && g_nregions < 64) g_regions[g_nregions++] = {reinterpret_cast<uintptr_t>(base), bytes};
}
extern "C" int sanitize_calls(void) { return g_calls; }
extern "C" int sanitize_violations(void) { return g_bad; }

namespace gdn {

hipError_t launch_gram(const GramArgs& a, int io, int nt, int nr, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.T * a.N * a.H * D * es_of(io);
  const int64_t mats = (int64_t)a.B * a.H * a.T * D * D * es_of(io);
  need(a.x0, tok, "gram x0");
  if (nr == 2) need(a.x1, tok, "gram x1");
  need(a.y, tok, "gram y");
  need(a.w, (int64_t)a.B * a.T * a.N * a.H * 4, "gram w");
  need(a.out0, mats, "gram out0");
  if (nr == 2) need(a.out1, mats, "gram out1");
  if (a.P > 1) need(a.part, (int64_t)a.P * a.B * a.H * a.Tc * nr * D * D * 4, "gram partials");
  return hipSuccess;
}
hipError_t launch_gram_reduce(const GramArgs& a, int io, int nt, int nr, hipStream_t s) {
  return launch_gram(a, io, nt, nr, s);
}
hipError_t launch_scan(const ScanArgs& a, int io, int nt, int mode, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt;
  const int64_t mats = (int64_t)a.B * a.H * a.T * D * D * es_of(io);
  need(a.A, mats, "scan A");
  need(a.U, mats, "scan U");
  need(a.gamma, (int64_t)a.B * a.T * a.H * 4, "scan gamma");
  need(a.z0, (int64_t)a.B * a.H * D * D * 4, "scan z0");
  // (with emit_entry the walk also writes the entering state one slot
  // before `emit`)
  need(a.emit_entry ? static_cast<const char*>(a.emit) - D * D * es_of(io) : a.emit, mats,
       "scan emit");
  need(a.zT, (int64_t)a.B * a.H * D * D * 4, "scan zT");
  const int ch = a.chunk > 0 ? a.chunk : a.Tc;
  const int64_t nck = (a.Tc + ch - 1) / ch;
  if (mode == SCAN_COMP_FWD || mode == SCAN_COMP_REV) {
    need(a.compC, (int64_t)a.B * a.H * nck * D * D * 4, "scan compC");
    need(a.compH, (int64_t)a.B * a.H * nck * D * D * 4, "scan compH");
  }
  if (a.chunk > 0 && a.zmid) need(a.zmid, (int64_t)a.B * a.H * nck * D * D * 4, "scan zmid");
  return hipSuccess;
}
hipError_t launch_output(const OutArgs& a, int io, int nt, bool, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.T * a.N * a.H * D * es_of(io);
  need(a.tok, tok, "output tok");
  need(a.mat, (int64_t)a.B * a.H * a.T * D * D * es_of(io), "output mat");
  need(a.out, tok, "output out");
  need(a.inv_out, (int64_t)a.B * a.T * a.N * a.H * 4, "output inv_out");
  return hipSuccess;
}
bool xdq_supported(int io, int64_t B, int64_t T, int64_t H) {
  return io == IO_BF16 && B * T * (H % 2 == 0 ? H / 2 : H) >= 256;
}
hipError_t launch_xdq(const XdqArgs& a, int io, int nt, hipStream_t) {
  // (the fused pass declines fp32 and launches of few items, like the real one)
  if (!xdq_supported(io, a.B, a.T, a.H)) return hipErrorNotSupported;
  ++g_calls;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.T * a.N * a.H * D * 2;
  const int64_t mats = (int64_t)a.B * a.H * a.T * D * D * 2;
  need(a.d_o, tok, "xdq d_o");
  need(a.q, tok, "xdq q");
  need(a.S, mats, "xdq S");
  need(a.X, mats, "xdq X");
  need(a.dq, tok, "xdq dq");
  need(a.inv, (int64_t)a.B * a.T * a.N * a.H * 4, "xdq inv");
  return hipSuccess;
}
hipError_t launch_dm(const DmArgs& a, int io, int nt, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt, mats = (int64_t)a.B * a.H * a.T * D * D * es_of(io);
  need(a.S, mats, "dm S");
  need(a.s0, (int64_t)a.B * a.H * D * D * 4, "dm s0");
  need(a.G, mats, "dm G");
  need(a.W, mats, "dm W");
  need(a.dgamma, (int64_t)a.B * a.T * a.H * 4, "dm dgamma");
  return hipSuccess;
}
hipError_t launch_bwd_tok(const BwdTokArgs& a, int io, int nt, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.T * a.N * a.H * D * es_of(io);
  const int64_t mats = (int64_t)a.B * a.H * a.T * D * D * es_of(io);
  need(a.k, tok, "bwd k");
  need(a.v, tok, "bwd v");
  need(a.beta, (int64_t)a.B * a.T * a.N * a.H * 4, "bwd beta");
  need(a.G, mats, "bwd G");
  need(a.W, mats, "bwd W");
  need(a.dk, tok, "bwd dk");
  need(a.dv, tok, "bwd dv");
  need(a.dbeta, (int64_t)a.B * a.T * a.N * a.H * 4, "bwd dbeta");
  need(a.S, mats, "bwd S");
  need(a.s0, (int64_t)a.B * a.H * D * D * 4, "bwd s0");
  need(a.dgamma, (int64_t)a.B * a.T * a.H * 4, "bwd dgamma");
  if (a.norm && io != gdn::IO_BF16) return hipErrorInvalidValue;
  return hipSuccess;
}
hipError_t launch_sigmoid(const float* x, float* y, int64_t n, hipStream_t) {
  ++g_calls;
  need(x, n * 4, "sigmoid x");
  need(y, n * 4, "sigmoid y");
  return hipSuccess;
}
hipError_t launch_sigmoid_bwd(const float* x, float* g, int64_t n, hipStream_t) {
  ++g_calls;
  need(x, n * 4, "sigmoid_bwd x");
  need(g, n * 4, "sigmoid_bwd g");
  return hipSuccess;
}
hipError_t launch_rows_normalize(const void* x, void* y, float* inv, int64_t rows, int d, int io,
                                 hipStream_t) {
  ++g_calls;
  need(x, rows * d * es_of(io), "rows_normalize x");
  need(y, rows * d * es_of(io), "rows_normalize y");
  need(inv, rows * 4, "rows_normalize inv");
  return hipSuccess;
}
hipError_t launch_rows_normalize_bwd(const void* x, void* g, int64_t rows, int d, int io,
                                     hipStream_t) {
  ++g_calls;
  need(x, rows * d * es_of(io), "rows_normalize_bwd x");
  need(g, rows * d * es_of(io), "rows_normalize_bwd g");
  return hipSuccess;
}
hipError_t launch_direct(const DirectArgs& a, int nt, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.T * a.N * a.H * D * 2;
  need(a.k, tok, "direct k");
  need(a.v, tok, "direct v");
  need(a.gamma, (int64_t)a.B * a.T * a.H * 4, "direct gamma");
  need(a.beta, (int64_t)a.B * a.T * a.N * a.H * 4, "direct beta");
  need(a.z0, (int64_t)a.B * a.H * D * D * 4, "direct z0");
  need(a.emit, (int64_t)a.B * a.H * a.T * D * D * 2, "direct emit");
  need(a.zT, (int64_t)a.B * a.H * D * D * 4, "direct zT");
  return hipSuccess;
}
hipError_t launch_direct_parts(const DirectArgs& a, int nt, hipStream_t) {
  ++g_calls;
  if (a.T != 1 || !a.part || a.P < 1) return hipErrorInvalidValue;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.N * a.H * D * 2;
  need(a.k, tok, "direct parts k");
  need(a.v, tok, "direct parts v");
  need(a.beta, (int64_t)a.B * a.N * a.H * 4, "direct parts beta");
  need(a.z0, (int64_t)a.B * a.H * D * D * 4, "direct parts z0");
  need(a.part, (int64_t)a.B * a.H * a.P * D * D * 4, "direct parts");
  return hipSuccess;
}
hipError_t launch_direct_out(const DirectArgs& a, int nt, hipStream_t) {
  ++g_calls;
  if (a.T != 1 || !a.part || a.P < 1 || !a.q || !a.o) return hipErrorInvalidValue;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.N * a.H * D * 2;
  need(a.q, tok, "direct out q");
  need(a.o, tok, "direct out o");
  need(a.gamma, (int64_t)a.B * a.H * 4, "direct out gamma");
  need(a.z0, (int64_t)a.B * a.H * D * D * 4, "direct out z0");
  need(a.zT, (int64_t)a.B * a.H * D * D * 4, "direct out zT");
  need(a.part, (int64_t)a.B * a.H * a.P * D * D * 4, "direct out parts");
  return hipSuccess;
}
hipError_t launch_token(const TokArgs& a, int io, int nt, bool, hipStream_t) {
  ++g_calls;
  const int64_t D = 16 * nt, tok = (int64_t)a.B * a.T * a.N * a.H * D * es_of(io);
  need(a.q, tok, "token q");
  need(a.k, tok, "token k");
  need(a.v, tok, "token v");
  need(a.o, tok, "token o");
  need(a.ws, (int64_t)a.B * a.H * a.nck * a.rec_bytes, "token records");
  if (a.mode == TOK_COMPOSITE) {
    need(a.compH, (int64_t)a.B * a.H * a.nseg * D * D * 4, "token compH");
    need(a.compC, (int64_t)a.B * a.H * a.nseg * D * D * 4, "token compC");
  }
  if (a.mode == TOK_REPLAY) need(a.zin, (int64_t)a.B * a.H * a.nseg * D * D * 4, "token zin");
  return hipSuccess;
}

}  // namespace gdn
