// Sanitizer driver for libgdn's host code: every entry point of include/gdn.h
// is called over a grid of problems with arguments that must pass
// validation (the launch stubs then check every device pointer against the
// regions handed in: tensors and the carved workspace) and with arguments
// that must be refused before any launch.  Device pointers are fake,
// well-separated addresses: the host code only does arithmetic on them.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host;
// exits non-zero on any failed expectation.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "gdn.h"
#include "sanitize_regions.h"

namespace {

int g_fail = 0;
long g_cases = 0;

#define EXPECT(cond, ...)                                            \
  do {                                                               \
    ++g_cases;                                                       \
    if (!(cond)) {                                                   \
      ++g_fail;                                                      \
      if (g_fail < 30) {                                             \
        fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);         \
        fprintf(stderr, __VA_ARGS__);                                \
        fprintf(stderr, "\n");                                       \
      }                                                              \
    }                                                                \
  } while (0)

// Fake device memory: region i starts at 2^44 + i 2^38 (far apart, 256-byte
// aligned); `slot` counts the regions of one call.
struct Fake {
  int slot = 0;
  void* take(int64_t bytes) {
    if (bytes <= 0) return nullptr;
    void* p = reinterpret_cast<void*>((uintptr_t(1) << 44) + (uintptr_t)(slot++) * (uintptr_t(1) << 38));
    sanitize_region(p, bytes);
    return p;
  }
};

gdn_problem make(int B, int H, int T, int N, int D, int io, int algo, int chunk, int flags) {
  gdn_problem p;
  memset(&p, 0, sizeof(p));
  p.B = B; p.H = H; p.T = T; p.N = N; p.Dk = D; p.Dv = D;
  p.io_dtype = io; p.key_scale = 0.f; p.scan_chunk = chunk; p.algorithm = algo; p.flags = flags;
  return p;
}

void run_valid(const gdn_problem& p) {
  const int64_t es = p.io_dtype == GDN_BF16 ? 2 : 4;
  const int64_t L = (int64_t)p.T * p.N;
  const int64_t tok = (int64_t)p.B * L * p.H * p.Dk * es;
  const int64_t gam = (int64_t)p.B * p.T * p.H * 4, bet = (int64_t)p.B * L * p.H * 4;
  const int64_t stb = (int64_t)p.B * p.H * p.Dk * p.Dk * 4;
  size_t wsf = 0, wsb = 0, sv = 0;
  EXPECT(gdn_workspace_size(&p, GDN_OP_FORWARD, &wsf) == GDN_OK, "workspace_size forward");
  EXPECT(gdn_workspace_size(&p, GDN_OP_BACKWARD, &wsb) == GDN_OK, "workspace_size backward");
  const bool has_saved = gdn_saved_size(&p, &sv) == GDN_OK;
  for (int variant = 0; variant < 4; ++variant) {
    const bool with_state = variant & 1, with_saved = (variant & 2) && has_saved;
    if ((variant & 2) && !has_saved) continue;
    sanitize_reset();
    Fake f;
    const void* q = f.take(tok); const void* k = f.take(tok); const void* v = f.take(tok);
    const float* g = (const float*)f.take(gam); const float* b = (const float*)f.take(bet);
    const float* s0 = with_state ? (const float*)f.take(stb) : nullptr;
    void* o = f.take(tok);
    float* sT = (float*)f.take(stb);
    void* saved = with_saved ? f.take((int64_t)sv) : nullptr;
    void* ws = f.take(wsf > 0 ? (int64_t)wsf : 16);
    int st = gdn_forward(&p, q, k, v, g, b, s0, o, sT, saved, ws, wsf > 0 ? wsf : 16, nullptr);
    EXPECT(st == GDN_OK, "forward B%d H%d T%d N%d D%d io%d algo%d chunk%d flags%d v%d: %s", p.B,
           p.H, p.T, p.N, p.Dk, p.io_dtype, p.algorithm, p.scan_chunk, p.flags, variant,
           gdn_status_string(st));
    EXPECT(sanitize_calls() > 0 && sanitize_violations() == 0,
           "forward launches: %d calls, %d out of bounds (B%d H%d T%d N%d D%d io%d algo%d)",
           sanitize_calls(), sanitize_violations(), p.B, p.H, p.T, p.N, p.Dk, p.io_dtype,
           p.algorithm);
    // in-place state
    if (with_state) {
      sanitize_reset();
      Fake f2;
      q = f2.take(tok); k = f2.take(tok); v = f2.take(tok);
      g = (const float*)f2.take(gam); b = (const float*)f2.take(bet);
      float* sio = (float*)f2.take(stb);
      o = f2.take(tok);
      ws = f2.take(wsf > 0 ? (int64_t)wsf : 16);
      st = gdn_forward(&p, q, k, v, g, b, sio, o, sio, nullptr, ws, wsf > 0 ? wsf : 16, nullptr);
      EXPECT(st == GDN_OK && sanitize_violations() == 0, "forward in place: %s",
             gdn_status_string(st));
    }
    // one frame too small a workspace: refused before any launch
    if (wsf > 0) {
      sanitize_reset();
      st = gdn_forward(&p, q, k, v, g, b, s0, o, sT, saved, ws, wsf - 1, nullptr);
      EXPECT(st == GDN_ERR_WORKSPACE_TOO_SMALL && sanitize_calls() == 0, "short workspace: %s",
             gdn_status_string(st));
    }
    // backward (the frame form; with or without the saved buffer)
    if (p.algorithm == GDN_ALGO_TOKEN || p.algorithm == GDN_ALGO_DIRECT) continue;
    sanitize_reset();
    Fake fb;
    q = fb.take(tok); k = fb.take(tok); v = fb.take(tok);
    g = (const float*)fb.take(gam); b = (const float*)fb.take(bet);
    s0 = with_state ? (const float*)fb.take(stb) : nullptr;
    const void* dO = fb.take(tok);
    const float* dsT = with_state ? (const float*)fb.take(stb) : nullptr;
    const void* sv_in = with_saved ? fb.take((int64_t)sv) : nullptr;
    void* dq = fb.take(tok); void* dk = fb.take(tok); void* dv = fb.take(tok);
    float* dg = (float*)fb.take(gam); float* db = (float*)fb.take(bet);
    float* ds0 = (float*)fb.take(stb);
    void* wb = fb.take((int64_t)wsb);
    st = gdn_backward(&p, q, k, v, g, b, s0, dO, dsT, sv_in, dq, dk, dv, dg, db, ds0, wb, wsb,
                      nullptr);
    EXPECT(st == GDN_OK && sanitize_calls() > 0 && sanitize_violations() == 0,
           "backward B%d H%d T%d N%d D%d io%d chunk%d flags%d saved%d: %s (%d calls, %d oob)", p.B,
           p.H, p.T, p.N, p.Dk, p.io_dtype, p.scan_chunk, p.flags, (int)with_saved,
           gdn_status_string(st), sanitize_calls(), sanitize_violations());
  }
  // the streaming step (one frame, state in place)
  if (p.T == 1) {
    size_t wss = 0;
    EXPECT(gdn_workspace_size(&p, GDN_OP_STEP, &wss) == GDN_OK, "workspace_size step");
    sanitize_reset();
    Fake f;
    const void* q = f.take(tok); const void* k = f.take(tok); const void* v = f.take(tok);
    const float* g = (const float*)f.take(gam); const float* b = (const float*)f.take(bet);
    float* sio = (float*)f.take(stb);
    void* o = f.take(tok);
    void* ws = f.take(wss > 0 ? (int64_t)wss : 16);
    const int st = gdn_step(&p, q, k, v, g, b, sio, o, ws, wss > 0 ? wss : 16, nullptr);
    EXPECT(st == GDN_OK && sanitize_violations() == 0, "step: %s", gdn_status_string(st));
  }
}

void run_invalid() {
  gdn_problem p = make(1, 2, 3, 5, 16, GDN_BF16, GDN_ALGO_AUTO, 0, 0);
  size_t n = 0;
  EXPECT(gdn_workspace_size(nullptr, GDN_OP_FORWARD, &n) == GDN_ERR_NULL_POINTER, "null problem");
  EXPECT(gdn_workspace_size(&p, GDN_OP_FORWARD, nullptr) == GDN_ERR_NULL_POINTER, "null size");
  EXPECT(gdn_workspace_size(&p, 7, &n) == GDN_ERR_BAD_SHAPE, "bad op");
  EXPECT(gdn_workspace_size(&p, GDN_OP_STEP, &n) == GDN_ERR_BAD_SHAPE, "step with T = 3");
  const int fields[][2] = {{0, 0}, {1, 0}, {2, 0}, {3, 0}, {0, -1}, {4, 24}, {4, 144}, {5, 32}};
  for (const auto& fv : fields) {
    gdn_problem b = p;
    int32_t* f[] = {&b.B, &b.H, &b.T, &b.N, &b.Dk, &b.Dv};
    *f[fv[0]] = fv[1];
    EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) != GDN_OK, "field %d = %d accepted", fv[0],
           fv[1]);
  }
  gdn_problem b = p;
  b.io_dtype = 5;
  EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) == GDN_ERR_BAD_DTYPE, "dtype");
  b = p; b.algorithm = 9;
  EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) == GDN_ERR_UNSUPPORTED, "algorithm");
  b = p; b.flags = 8;
  EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) == GDN_ERR_UNSUPPORTED, "flags");
  b = p; b.key_scale = 1.f / 0.f;
  EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) == GDN_ERR_BAD_SHAPE, "infinite scale");
  b = make(1 << 20, 1 << 10, 1 << 10, 1, 16, GDN_BF16, 0, 0, 0);
  EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) == GDN_ERR_BAD_SHAPE, "grid overflow");
  b = make(1, 1, 1, 1 << 24, 16, GDN_BF16, 0, 0, 0);
  EXPECT(gdn_workspace_size(&b, GDN_OP_FORWARD, &n) == GDN_ERR_BAD_SHAPE, "N at 2^24");

  // pointers: null, misaligned, aliasing, all before any launch
  sanitize_reset();
  Fake f;
  const int64_t tok = 1 * 15 * 2 * 16 * 2;
  char* q = (char*)f.take(tok); char* k = (char*)f.take(tok); char* v = (char*)f.take(tok);
  float* g = (float*)f.take(64); float* be = (float*)f.take(256);
  char* o = (char*)f.take(tok);
  size_t wsf = 0;
  gdn_workspace_size(&p, GDN_OP_FORWARD, &wsf);
  char* ws = (char*)f.take((int64_t)wsf + 64);
  EXPECT(gdn_forward(&p, nullptr, k, v, g, be, nullptr, o, nullptr, nullptr, ws, wsf, nullptr) ==
             GDN_ERR_NULL_POINTER, "null q");
  EXPECT(gdn_forward(&p, q + 2, k, v, g, be, nullptr, o, nullptr, nullptr, ws, wsf, nullptr) ==
             GDN_ERR_MISALIGNED, "misaligned q");
  EXPECT(gdn_forward(&p, q, k, v, (float*)((char*)g + 2), be, nullptr, o, nullptr, nullptr, ws,
                     wsf, nullptr) == GDN_ERR_MISALIGNED, "misaligned gamma");
  EXPECT(gdn_forward(&p, q, k, v, g, be, nullptr, q, nullptr, nullptr, ws, wsf, nullptr) ==
             GDN_ERR_ALIASING, "o aliases q");
  EXPECT(gdn_forward(&p, q, k, v, g, be, nullptr, o, nullptr, nullptr, k, wsf, nullptr) ==
             GDN_ERR_ALIASING, "workspace aliases k");
  EXPECT(gdn_forward_events(&p, q, k, v, g, be, nullptr, o, nullptr, nullptr, ws, wsf, nullptr,
                            nullptr) == GDN_ERR_NULL_POINTER, "null events");
  EXPECT(sanitize_calls() == 0, "a refused call launched something");
  // backward: a dbeta that overlaps beta is refused
  size_t wsb = 0;
  gdn_workspace_size(&p, GDN_OP_BACKWARD, &wsb);
  char* wb = (char*)f.take((int64_t)wsb);
  char* dO = (char*)f.take(tok); char* dq = (char*)f.take(tok); char* dk = (char*)f.take(tok);
  char* dv = (char*)f.take(tok); float* dg = (float*)f.take(64);
  EXPECT(gdn_backward(&p, q, k, v, g, be, nullptr, dO, nullptr, nullptr, dq, dk, dv, dg, be,
                      nullptr, wb, wsb, nullptr) == GDN_ERR_ALIASING, "dbeta aliases beta");
  EXPECT(sanitize_calls() == 0, "a refused backward launched something");
  // the static-scratch forward: a problem beyond its scratch
  gdn_problem big = make(1, 20, 121, 880, 112, GDN_FP32, 0, 0, 0);
  EXPECT(gdn_forward_noalloc(&big, q, k, v, g, be, nullptr, o, nullptr, nullptr, nullptr) ==
             GDN_ERR_SCRATCH_TOO_SMALL, "noalloc beyond its scratch");
  EXPECT(gdn_abi_version() == GDN_ABI_VERSION, "abi version");
  for (int c = -1; c < 12; ++c) EXPECT(gdn_status_string(c) != nullptr, "status string");
}

// The stubs' bounds check itself: the same call, with the workspace region
// registered one byte short of what the call may use, must be flagged.
void negative_control() {
  const gdn_problem p = make(1, 4, 6, 40, 48, GDN_BF16, GDN_ALGO_FRAME, 0, 0);
  const int64_t tok = (int64_t)6 * 40 * 4 * 48 * 2;
  size_t wsf = 0;
  gdn_workspace_size(&p, GDN_OP_FORWARD, &wsf);
  sanitize_reset();
  Fake f;
  const void* q = f.take(tok); const void* k = f.take(tok); const void* v = f.take(tok);
  const float* g = (const float*)f.take(6 * 4 * 4);
  const float* b = (const float*)f.take(240 * 4 * 4);
  void* o = f.take(tok);
  void* ws = f.take((int64_t)wsf - 1);
  const int st = gdn_forward(&p, q, k, v, g, b, nullptr, o, nullptr, nullptr, ws, wsf, nullptr);
  EXPECT(st == GDN_OK && sanitize_violations() > 0,
         "a workspace one byte short went unnoticed by the stubs (%d violations)",
         sanitize_violations());
}

}  // namespace

int main() {
  negative_control();
  run_invalid();
  const int Bs[] = {1, 2}, Hs[] = {1, 2, 3, 20}, Ts[] = {1, 2, 5, 121}, Ns[] = {1, 7, 33, 880};
  const int Ds[] = {16, 48, 112, 128};
  long valid = 0;
  for (int B : Bs)
    for (int H : Hs)
      for (int T : Ts)
        for (int N : Ns)
          for (int D : Ds)
            for (int io = 0; io < 2; ++io)
              for (int algo = 0; algo < 4; ++algo)
                for (int chunk : {0, 1, 3})
                  for (int flags = 0; flags < 4; ++flags) {
                    // a subsample of the full product, every value of every axis present
                    if ((B * 7 + H * 5 + T * 3 + N + D + io * 11 + algo * 13 + chunk * 17 +
                         flags * 19) % 5 != 0)
                      continue;
                    const gdn_problem p = make(B, H, T, N, D, io, algo, chunk, flags);
                    size_t n = 0;
                    if (gdn_workspace_size(&p, GDN_OP_FORWARD, &n) != GDN_OK) continue;
                    ++valid;
                    run_valid(p);
                  }
  printf("sanitize driver: %ld valid problems, %ld expectations, %d failed\n", valid, g_cases,
         g_fail);
  return g_fail == 0 ? 0 : 1;
}
