/*
 * libgdn: frame-wise Gated DeltaNet (GDN) token mixer for MI355X (gfx950).
 *
 * The operation (paper.rainbus.top summary of "SANA-WM: Efficient
 * Minute-Scale World Modeling with Hybrid Linear Diffusion Transformer"):
 *   - section 前置知识, "Gated DeltaNet (GDN)": one D x D state S_t per head,
 *     S_t = S_{t-1} M_t + U_t;
 *   - section 方法步骤详情, module 2: the scan advances once per latent frame,
 *       M_t = gamma_t I - K^_t beta_t K^_t^T,  U_t = V_t beta_t K^_t^T,
 *       O_t = S_t Q^_t,
 *     with keys scaled by 1/sqrt(D S) (D = head dim, S = tokens per frame);
 *   - section 技术新颖性, point 1: the frame-wise scan generalises token-wise
 *     GDN; transition composites C_p and input composites H_p combine by a
 *     prefix that reproduces the sequential result exactly.
 * Column form: K^_t, Q^_t are D x N (a column per token), V_t, O_t are D x N,
 * beta_t = diag(beta_t1 .. beta_tN), S is Dv x Dk (row i = value dim i).
 *
 * Memory layout (row-major, contiguous, frame-major tokens l = t*N + n):
 *   q, k            [B, L, H, Dk]    io dtype (bf16 or fp32)
 *   v, o, d_o       [B, L, H, Dv]    io dtype
 *   gamma           [B, T, H]        fp32   (one decay per frame and head)
 *   beta            [B, L, H]        fp32   (one write strength per token)
 *   state_*         [B, H, Dv, Dk]   fp32
 *   dgamma [B,T,H], dbeta [B,L,H]    fp32
 * By default queries and keys are used as given (the library applies only
 * the key scale) and gamma, beta are the gates themselves; the problem's
 * `flags` can ask for the block's prologue instead (gdn_flag).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after returning.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).
 *     Nothing synchronises the device.
 *   - Arguments are validated on the host before any launch.  On a
 *     validation error nothing is launched, nothing is written, and a
 *     specific gdn_status is returned.  A failed launch returns
 *     GDN_ERR_HIP (outputs then undefined).  Device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.
 *   - Tensor and workspace pointers must be 16-byte aligned; the gate
 *     pointers (gamma, beta, dgamma, dbeta) 4-byte aligned.  Outputs must
 *     not overlap inputs, except where an entry point says so.
 *   - Reentrant: no mutable global state, except the static scratch that
 *     gdn_forward_noalloc shares between its calls on one GPU.
 *   - Supported shapes: Dk == Dv == D with D a multiple of 16 and <= 128;
 *     B, H, T, N >= 1; B*H*T must fit in int32 and B*L*H be at most 2^40;
 *     one frame's token rows (N*H*D io elements) under 2 GiB, and N and
 *     H*D*(io element bytes) under 2^24.  Other sizes: GDN_ERR_BAD_SHAPE.
 */
#ifndef LIBGDN_GDN_H
#define LIBGDN_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 4

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_POINTER = 1,        /* a required pointer is NULL            */
    GDN_ERR_BAD_SHAPE = 2,           /* a size < 1 or inconsistent            */
    GDN_ERR_BAD_DTYPE = 3,           /* io_dtype not a gdn_dtype              */
    GDN_ERR_MISALIGNED = 4,          /* a pointer misaligned (16 B; gates 4 B) */
    GDN_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < required            */
    GDN_ERR_UNSUPPORTED = 6,         /* D not a multiple of 16, > 128, Dk!=Dv;
                                        unknown algorithm or flag; token or
                                        direct form outside its limits
                                        (gdn_algorithm)                       */
    GDN_ERR_HIP = 7,                 /* a kernel launch failed                */
    GDN_ERR_ALIASING = 8,            /* an output overlaps an input           */
    GDN_ERR_SCRATCH_TOO_SMALL = 9    /* gdn_forward_noalloc: the problem needs
                                        more than GDN_NOALLOC_SCRATCH_BYTES  */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_FP32 = 1 } gdn_dtype;

typedef enum { GDN_OP_FORWARD = 0, GDN_OP_STEP = 1, GDN_OP_BACKWARD = 2 } gdn_op;

/* How gdn_forward / gdn_step evaluate the recurrence (same result up to
 * rounding order):
 *   GDN_ALGO_FRAME  the frame form: per frame A_t = K^_t beta_t K^_t^T and
 *                   U_t = V_t beta_t K^_t^T (D x D), a scan over frames,
 *                   then O_t = S_t Q^_t.  Any N.  Fills `saved`.
 *   GDN_ALGO_TOKEN  the token form: chunks of F = floor(64 / N) frames
 *                   (bf16; 32 / N for fp32) whose corrected values solve the
 *                   delta rule's unit triangular system over the chunk's
 *                   tokens; no D x D product per frame.  Its workspace
 *                   holds each chunk's operators (17.25 KiB per chunk,
 *                   head and batch in bf16).  For frames of few tokens
 *                   (token-wise GDN is N = 1).
 *                   Requires N <= 64 (bf16) / 32 (fp32) and saved == NULL.
 *   GDN_ALGO_DIRECT the direct form: the frames in turn in one launch,
 *                   S_t = gamma_t S_{t-1} + sum_n beta_n (s v_n -
 *                   s^2 S_{t-1} k_n) k_n^T straight from the token rows
 *                   (no A_t, U_t), then O_t = S_t Q^_t for all frames.
 *                   For launches of few frames (streaming steps, short
 *                   windows).  A launch of one frame of 129 to 4096 tokens
 *                   splits the frame's tokens into parts of 128, each
 *                   part's update kept in fp32 in the workspace (B H D^2 4
 *                   bytes a part) and summed in a fixed order.  bf16 only;
 *                   requires saved == NULL.
 *   GDN_ALGO_AUTO   the direct form for bf16 launches of at most 2 frames
 *                   (the frame form when a saved buffer is passed), else
 *                   the frame form.
 * gdn_backward always uses the frame form (recomputing A_t, S_t when no
 * saved buffer is given). */
typedef enum {
    GDN_ALGO_AUTO = 0, GDN_ALGO_FRAME = 1, GDN_ALGO_TOKEN = 2, GDN_ALGO_DIRECT = 3
} gdn_algorithm;

/* Optional prologue of the GDN block, fused into the entry points (bits of
 * gdn_problem.flags; any other bit is GDN_ERR_UNSUPPORTED).  The hats on
 * Q^_t and K^_t (summary page, 方法步骤详情 module 2) read as per-token
 * normalisation:
 *   GDN_FLAG_NORMALIZE_QK  every query and key row (one token, one head) is
 *                          divided by its L2 norm over the head dimension
 *                          before the key scale; a row of zeros stays zero.
 *                          The frame form's forward takes the norms from the
 *                          rows it already stages (no extra pass over q, k).
 *   GDN_FLAG_GATE_LOGITS   gamma and beta arrive as logits x and the
 *                          recurrence uses sigmoid(x) = 1 / (1 + exp(-x)).
 * gdn_backward then returns the gradients with respect to these raw inputs
 * (chain rule through the prologue). */
typedef enum { GDN_FLAG_NORMALIZE_QK = 1, GDN_FLAG_GATE_LOGITS = 2 } gdn_flag;

typedef struct {
    int32_t B, H, T, N;   /* batch, heads, latent frames, tokens per frame   */
    int32_t Dk, Dv;       /* head dims; must be equal                        */
    int32_t io_dtype;     /* gdn_dtype of q, k, v, o, d_o, dq, dk, dv        */
    float key_scale;      /* 0 => 1/sqrt(Dk * N), the 1/sqrt(D S) of the
                             summary page (module 2; novelty point 1)        */
    int32_t scan_chunk;   /* inter-frame scan: 0 => library default (chunks
                             of 16 frames for at most 8 sequences B H, 32
                             for at most 16, else sequential),
                             1 => sequential over frames,
                             c >= 2 => composite prefix over chunks of c
                             frames (novelty point 1); same result up to
                             rounding order                                  */
    int32_t algorithm;    /* gdn_algorithm of the forward                    */
    int32_t flags;        /* OR of gdn_flag; 0 => no prologue                */
} gdn_problem;

/* Version of this interface (GDN_ABI_VERSION). */
int gdn_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* gdn_status_string(int status);

/* Bytes of device workspace the entry point `op` needs for problem `p`
 * (written to *bytes).  0 is a valid answer.  Validates `p` like the
 * entry point does. */
gdn_status gdn_workspace_size(const gdn_problem* p, int op, size_t* bytes);

/* Bytes of the optional forward->backward buffer `saved` (written to
 * *bytes).  Layout: A_t = K^_t beta_t K^_t^T as [B, H, T] x Dk x Dk,
 * followed by the states S_t after every frame as [B, H, T, Dv, Dk]
 * row-major, in the intermediate type: bf16 (round to nearest even) when
 * io_dtype is GDN_BF16, fp32 when it is GDN_FP32; with
 * GDN_FLAG_NORMALIZE_QK then 1 / |q| of every query row as fp32 [B, L, H]
 * (0 for a zero row), which the output pass forms anyway and the backward
 * reads instead of a pass over q.  fp32 A_t is row-major;
 * bf16 A_t is in the MFMA operand order of the scan: element [r][c] of a
 * frame's A_t at (r / 16) 16 Dk + (c / 32) 512 + (16 ((c % 32) / 8) +
 * r % 16) 8 + c % 8.  GDN_ERR_UNSUPPORTED for GDN_ALGO_TOKEN and
 * GDN_ALGO_DIRECT, which keep neither. */
gdn_status gdn_saved_size(const gdn_problem* p, size_t* bytes);

/* Whole-sequence forward (module 2 recurrence over t = 1..T):
 *   S_t = S_{t-1} (gamma_t I - K^_t beta_t K^_t^T) + V_t beta_t K^_t^T,
 *   O_t = S_t Q^_t,  K^ = key_scale * K,  Q^ = Q
 * (with GDN_FLAG_NORMALIZE_QK: K^ = key_scale * K / |K|, Q^ = Q / |Q| per
 * row; with GDN_FLAG_GATE_LOGITS gamma, beta are logits, see gdn_flag).
 *   state_in   S_0; NULL => zero.
 *   o          output [B, L, H, Dv], io dtype.
 *   state_out  S_T; NULL => not written; may equal state_in (in place).
 *   saved      NULL, or gdn_saved_size bytes that receive A_t and S_t for
 *              gdn_backward.
 *   workspace  gdn_workspace_size(p, GDN_OP_FORWARD) bytes of scratch. */
gdn_status gdn_forward(const gdn_problem* p,
                       const void* q, const void* k, const void* v,
                       const float* gamma, const float* beta,
                       const float* state_in,
                       void* o, float* state_out, void* saved,
                       void* workspace, size_t workspace_bytes, void* stream);

/* gdn_forward, additionally recording four caller-created hipEvent_t
 * (events[0..3], all non-NULL) on `stream`: before the per-frame Gram/write
 * kernel, between it and the inter-frame scan, between the scan and the
 * output kernel, and after the output kernel.  For measuring the three
 * phases; results are identical to gdn_forward.  The token form counts
 * entirely as the output phase; the direct form's state update as the
 * scan phase. */
gdn_status gdn_forward_events(const gdn_problem* p,
                              const void* q, const void* k, const void* v,
                              const float* gamma, const float* beta,
                              const float* state_in,
                              void* o, float* state_out, void* saved,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void* const* events);

/* Bytes of the static scratch of gdn_forward_noalloc (192 MiB): enough for
 * the forward's workspace at 20 heads x 112, 121 frames x 880 tokens in
 * bf16, prologue flags included. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)

/* gdn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * errors as gdn_forward, except that the workspace is the library's own
 * static scratch on the current device (hipGetDevice; `stream` must belong
 * to that device): one GDN_NOALLOC_SCRATCH_BYTES array per GPU, created with
 * the library's device code and held until the process ends.  Its device
 * address is looked up once per device, on the first call there.
 *   - A problem whose gdn_workspace_size(p, GDN_OP_FORWARD) exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_SCRATCH_TOO_SMALL before any
 *     GPU work.
 *   - Nothing is allocated or freed (no hipMalloc, hipFree or allocating
 *     library routine); nothing in the scratch needs to start at zero.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *     time on one GPU (other streams, other threads) race and corrupt each
 *     other's results.  Serialise them, e.g. on one stream.
 *   - GDN_ERR_HIP if the scratch's device address cannot be obtained. */
gdn_status gdn_forward_noalloc(const gdn_problem* p,
                               const void* q, const void* k, const void* v,
                               const float* gamma, const float* beta,
                               const float* state_in,
                               void* o, float* state_out, void* saved, void* stream);

/* Streaming step: advance the carried state by one latent frame
 * (p->T must be 1), as the chunk-by-chunk autoregressive variant does
 * (CSDN explainer section 六, stage 4).  `state` [B, H, Dv, Dk] is read as
 * S_{t-1} and overwritten with S_t; o receives O_t [B, N, H, Dv]. */
gdn_status gdn_step(const gdn_problem* p,
                    const void* q, const void* k, const void* v,
                    const float* gamma, const float* beta,
                    float* state, void* o,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Reverse pass of gdn_forward (the pages give none; chain rule of the
 * module-2 recurrence).  With G_t = dLoss/dS_t:
 *   G_T = dO_T Q^_T^T + dS_T,   G_t = dO_t Q^_t^T + G_{t+1} M_{t+1}^T,
 *   dQ^_t = S_t^T dO_t,  dM_t = S_{t-1}^T G_t,  dgamma_t = tr(dM_t),
 *   dV_t = G_t K^_t beta_t,
 *   dK_t = key_scale (G_t^T V_t beta_t - (dM_t + dM_t^T) K^_t beta_t),
 *   dbeta_tn = v_tn^T G_t k^_tn - k^_tn^T dM_t k^_tn,  dS_0 = G_1 M_1^T.
 *   state_in     S_0 of the forward; NULL => zero.
 *   d_o          [B, L, H, Dv] io dtype.
 *   d_state_out  dLoss/dS_T; NULL => zero.
 *   saved        the buffer gdn_forward filled for the same inputs, or
 *                NULL to recompute it inside the workspace.
 *   dq, dk, dv   io dtype, layouts of q, k, v.  dgamma, dbeta fp32.
 *   d_state_in   dLoss/dS_0; NULL => not written.
 *   workspace    gdn_workspace_size(p, GDN_OP_BACKWARD) bytes.
 * With p->flags set, q, k, gamma, beta are the raw inputs of the forward
 * and dq, dk, dgamma, dbeta the gradients with respect to them:
 * dx = (dx^ - x^ (x^ . dx^)) / |x| for a normalised row x^ = x / |x| (0 for
 * a zero row), dz = dp p (1 - p) for a gate p = sigmoid(z). */
gdn_status gdn_backward(const gdn_problem* p,
                        const void* q, const void* k, const void* v,
                        const float* gamma, const float* beta,
                        const float* state_in,
                        const void* d_o, const float* d_state_out,
                        const void* saved,
                        void* dq, void* dk, void* dv,
                        float* dgamma, float* dbeta, float* d_state_in,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN_GDN_H */
