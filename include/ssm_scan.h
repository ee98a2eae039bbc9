/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) S6 selective-scan library (libssm57.so).
 *
 * The operation (Mamba paper, arXiv 2312.00752, gitcode.csdn.net translation: section 2 "discretisation",
 * "computation" and "structure and dimensions"; section 3.2 (s_B, s_C, s_Delta, tau_Delta = softplus); section 3.3.2
 * (fused selective scan that never materialises the (B, L, D, N) state); docs.ifdog.com Mamba tutorial: "离散化"
 * (ZOH, diagonal A), "Mamba：选择性状态空间模型" (softplus, input-dependent B/C/Delta), "Mamba 架构" (SiLU gate)):
 *
 *   for every batch b and channel d independently, with a diagonal state h[0..N-1]:
 *     Delta_t = softplus(dt[b,d,t] + dt_bias[d])      (or dt + dt_bias when dt_softplus == 0)
 *     h[n]   <- exp(Delta_t * A[d,n]) * h[n] + Bbar_t[n] * x[b,d,t]
 *               Bbar_t[n] = Delta_t * B[b,n,t]                         (SSM_DISC_EULER_B, default)
 *               Bbar_t[n] = expm1(Delta_t*A[d,n]) / A[d,n] * B[b,n,t]  (SSM_DISC_ZOH; A == 0 uses Delta_t * B)
 *     y[b,d,t] = (sum_n C[b,n,t] * h[n] + Dskip[d] * x[b,d,t]) * silu(z[b,d,t]),  silu(v) = v * sigmoid(v)
 *   h starts at h0[b,d,:] (zeros when h0 == NULL) and its last value is written to h_final.
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE memory owned by the caller.  The library allocates nothing; the forward scan may
 *     need, and the backward always needs, a caller-provided workspace (query its size first).
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the default stream).  Buffers must stay
 *     alive until the stream has executed the call.  Nothing is synchronised implicitly.
 *   - Layouts are row-major with the sequence index innermost:  x, dt, z, y: [batch][dim][seqlen];
 *     B, C: [batch][dstate][seqlen];  A: [dim][dstate];  dt_bias, Dskip: [dim];  h0, h_final, state: [batch][dim][dstate].
 *     Decode tensors drop the seqlen axis: x, dt, z, y: [batch][dim];  B, C: [batch][dstate].
 *   - x, dt, B, C, z use params.io_dtype (fp32, or bf16 stored as its 16-bit pattern); y uses params.y_dtype;
 *     A, dt_bias, Dskip, h0, h_final, state and the arithmetic are fp32.  bf16 outputs are rounded to nearest-even.
 *   - Argument errors are reported BEFORE anything is launched: a non-OK status means no kernel ran and no output was
 *     touched.  Launch failures report SSM_ERR_HIP.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation, as with any asynchronous HIP work.  Non-finite inputs are not checked; they propagate.
 *   - y must not overlap any input.  h_final may alias h0.  The decode state is updated in place.
 *   - Results are deterministic: the same inputs and parameters give bit-identical outputs on every run.
 *   - Every function is reentrant; ssm_last_error() is thread-local.
 */
#ifndef SSM57_SSM_SCAN_H
#define SSM57_SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM57_ABI_VERSION 1
#define SSM57_MAX_DSTATE 16

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,         /* a required pointer is NULL */
  SSM_ERR_SHAPE = 2,        /* batch/dim/seqlen < 1, dstate outside [1, 16], batch > 65535, seqlen > 2^25
                               (32-bit per-lane offsets), sizes that overflow the grid (SSD limits: ssm_ssd_fwd) */
  SSM_ERR_DTYPE = 3,        /* unknown io_dtype / y_dtype */
  SSM_ERR_UNSUPPORTED = 4,  /* unknown disc or dt_softplus value, negative segments */
  SSM_ERR_ALIGN = 5,        /* a pointer not aligned to its element size */
  SSM_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than ssm_scan_{fwd,bwd}_workspace_bytes() */
  SSM_ERR_HIP = 7           /* the HIP runtime refused a launch */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

typedef enum {
  SSM_DISC_EULER_B = 0, /* Abar = exp(Delta A), Bbar = Delta B (the tutorial's simplified selective SSM) */
  SSM_DISC_ZOH = 1      /* Abar = exp(Delta A), Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B  (paper eq. (4)) */
} ssm_disc;

typedef struct {
  int64_t batch;       /* b >= 1 */
  int64_t dim;         /* D >= 1 channels (d_inner) */
  int64_t seqlen;      /* L >= 1 (ignored by ssm_state_update) */
  int64_t dstate;      /* N, 1 <= N <= 16 */
  int32_t io_dtype;    /* ssm_dtype of x, dt, B, C, z */
  int32_t y_dtype;     /* ssm_dtype of y */
  int32_t disc;        /* ssm_disc */
  int32_t dt_softplus; /* 1: Delta = softplus(dt + dt_bias); 0: Delta = dt + dt_bias */
  int32_t segments;    /* 0: the library picks the number of L-segments scanned in parallel; k > 0 forces k
                          (clamped to the number of 64-step chunks); results agree within rounding either way */
  int32_t reserved;    /* must be 0 */
} ssm_scan_params;

/*
 * Causal depthwise convolution in front of the scan (the Mamba block's SSM branch: docs.ifdog.com tutorial, "Mamba 架构"
 * step 3a -- a 1-D causal convolution of kernel size d_conv, usually 4, each channel on its own -- followed by the
 * block's SiLU activation, Mamba paper section 3.4).  With it the scan's input x is replaced by
 *   u[b,d,t] = act(bias[d] + sum_{k=0}^{width-1} weight[d][k] * x[b,d,t-(width-1)+k]),   act = SiLU or identity,
 * where x before t = 0 comes from state_in (oldest first; zeros when NULL).  u feeds both the recurrence and the D
 * skip; it is computed in the scan kernel and never written to memory.
 */
typedef struct {
  const float* weight;   /* [dim][width] fp32, required */
  const float* bias;     /* [dim] fp32 or NULL (= 0) */
  const float* state_in; /* [batch][dim][width-1] fp32 or NULL (= zeros): the inputs before the first step */
  float* state_out;      /* [batch][dim][width-1] fp32 or NULL: the last width-1 inputs (continuing state_in when
                            seqlen < width-1), oldest first; may alias state_in */
  int32_t width;         /* 1 <= width <= 4 */
  int32_t activation;    /* 1: SiLU after the convolution; 0: none */
} ssm_conv_params;

/* Bytes of device workspace ssm_scan_fwd needs for these parameters (0 when none).  Pure host function.
 * ssm_conv_scan_fwd needs the same workspace. */
size_t ssm_scan_fwd_workspace_bytes(const ssm_scan_params* p);

/*
 * Full-sequence forward scan (steps: softplus Delta, discretisation, recurrence, C-contraction, D skip, SiLU gate).
 *   x, dt [batch][dim][seqlen] io_dtype;  dt_bias [dim] fp32 or NULL (= 0);  A [dim][dstate] fp32 (the diagonal of A;
 *   the method expects negative reals, not checked);  B, C [batch][dstate][seqlen] io_dtype;  Dskip [dim] fp32 or NULL
 *   (= no skip);  z [batch][dim][seqlen] io_dtype or NULL (= no gate);  h0 [batch][dim][dstate] fp32 or NULL (= 0);
 *   y [batch][dim][seqlen] y_dtype (written);  h_final [batch][dim][dstate] fp32 or NULL (written; may alias h0);
 *   workspace: device buffer of at least ssm_scan_fwd_workspace_bytes(p) bytes, 4-byte aligned (NULL if 0 needed);
 *   stream: hipStream_t or NULL.
 */
ssm_status ssm_scan_fwd(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* Dskip, const void* z, const float* h0, void* y,
                        float* h_final, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_fwd for callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without the workspace, which is instead a static 64 MiB device array of the
 * library (one per GPU, held until the process ends).  Nothing is allocated by the call.  When the segmented scan's
 * workspace would exceed 64 MiB, the correction window of each L-segment shrinks (down to 64 steps) until it fits,
 * so results may differ from ssm_scan_fwd's within rounding; SSM_ERR_SHAPE when even that does not fit (more than
 * about 64 MiB / (4 * (64 + 3 * dstate + 3)) segment-channel pairs).  All calls on one GPU share the array: calls that
 * overlap on the same GPU (different streams or host threads of one process) race and must be serialised by the caller.
 * Other errors as for ssm_scan_fwd; SSM_ERR_HIP if the array's device address cannot be obtained.
 */
ssm_status ssm_scan_fwd_noalloc(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias,
                                const float* A, const void* B, const void* C, const float* Dskip, const void* z,
                                const float* h0, void* y, float* h_final, void* stream);

/*
 * Single-token recurrent decode step (constant time and state per token; paper section 1 (ii) and section 2
 * "recurrent mode (2) for autoregressive inference").  Same arithmetic as one step of ssm_scan_fwd.
 *   state [batch][dim][dstate] fp32, read and overwritten in place;  x, dt, z, y [batch][dim];  B, C [batch][dstate];
 *   dt_bias, A, Dskip as above.  p->seqlen and p->segments are ignored.
 */
ssm_status ssm_state_update(const ssm_scan_params* p, float* state, const void* x, const void* dt,
                            const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                            const void* z, void* y, void* stream);

/*
 * ssm_scan_fwd with the causal convolution (+ activation) above applied to x first.  x [batch][dim][seqlen] io_dtype
 * is the convolution's input; every other argument is as for ssm_scan_fwd.  conv->state_out, if given, is written
 * after the scan has read conv->state_in, so the two may alias.
 */
ssm_status ssm_conv_scan_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* dt,
                             const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                             const void* z, const float* h0, void* y, float* h_final, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * ssm_state_update with the causal convolution: the convolution window of the last width-1 inputs is read from
 * conv->state_in and the shifted window (ending with this step's x) written to conv->state_out (both required for
 * width > 1; they may alias, which updates the window in place).  One step of ssm_conv_scan_fwd.
 */
ssm_status ssm_conv_state_update(const ssm_scan_params* p, const ssm_conv_params* conv, float* state, const void* x,
                                 const void* dt, const float* dt_bias, const float* A, const void* B, const void* C,
                                 const float* Dskip, const void* z, void* y, void* stream);

/*
 * The convolution above on its own, for training: u = act(bias + sum_k weight[k] x_{t-(width-1)+k}) with the inputs
 * before t = 0 from conv->state_in (conv->state_out is ignored).  A backward pass calls it to recompute u for
 * ssm_scan_bwd (which returns dL/du as its dx), then ssm_conv1d_bwd.  x [batch][dim][seqlen] io_dtype, u the same
 * shape in y_dtype.  p->dstate, disc and dt_softplus are validated as for the scan and otherwise unused.
 */
ssm_status ssm_conv1d_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, void* u,
                          void* stream);

/*
 * Backward of the convolution (+ activation): the chain rule through u above for the loss whose gradient is
 * du = dL/du [batch][dim][seqlen] y_dtype and, optionally, dstate_out = dL/d(conv->state_out) [batch][dim][width-1]
 * fp32 (the returned window).  Outputs (overwritten): dx [batch][dim][seqlen] y_dtype;  dweight [dim][width] fp32
 * (summed over batch and time, required);  dbias [dim] fp32 and dstate_in [batch][dim][width-1] fp32 (the incoming
 * window's gradient), each optional.  x, conv->weight, bias and state_in as given to the forward.  Deterministic.
 */
ssm_status ssm_conv1d_bwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* du,
                          const float* dstate_out, void* dx, float* dweight, float* dbias, float* dstate_in,
                          void* stream);

/*
 * Scan with a complex diagonal A (Mamba paper section 3.6 "real vs. complex", S4D-Lin initialisation A_n = -1/2 + n i,
 * used for continuous modalities such as audio, section 4.4).  The state is complex and so are B and C; the output
 * is real:  Abar = exp(Delta A),  Bbar = Delta B (SSM_DISC_EULER_B) or (exp(Delta A) - 1) / A * B (SSM_DISC_ZOH; A = 0
 * gives Delta B),  h_t = Abar h_{t-1} + Bbar x_t,  y_t = (Re(sum_n C_n(t) h_n(t)) + Dskip x_t) * silu(z_t).
 * Complex arrays are interleaved (re, im) pairs:  A [dim][dstate][2] fp32;  B, C [batch][dstate][seqlen][2] io_dtype;
 * h0, h_final [batch][dim][dstate][2] fp32.  x, dt, z, y, dt_bias, Dskip as for ssm_scan_fwd.  No workspace;
 * p->segments is ignored.
 */
ssm_status ssm_complex_scan_fwd(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias,
                                const float* A, const void* B, const void* C, const float* Dskip, const void* z,
                                const float* h0, void* y, float* h_final, void* stream);

/* One decode step of ssm_complex_scan_fwd: state [batch][dim][dstate][2] fp32 updated in place; x, dt, z, y
 * [batch][dim]; B, C [batch][dstate][2] io_dtype. */
ssm_status ssm_complex_state_update(const ssm_scan_params* p, float* state, const void* x, const void* dt,
                                    const float* dt_bias, const float* A, const void* B, const void* C,
                                    const float* Dskip, const void* z, void* y, void* stream);

/* Bytes of device workspace ssm_scan_bwd needs for these parameters (always > 0 for valid parameters, 0 for invalid
 * ones).  Pure host function. */
size_t ssm_scan_bwd_workspace_bytes(const ssm_scan_params* p);

/*
 * Backward of ssm_scan_fwd: the gradients of a scalar loss given dL/dy and, optionally, dL/dh_final.  They are the
 * chain rule through the operation above.  No state from the forward pass is needed: every intermediate state is
 * recomputed from the inputs (Mamba paper, gitcode.csdn.net translation, section 3.3.2, the recomputation paragraph;
 * alishangtian.com close reading, "hardware-aware algorithm", recomputation item).
 *   Parameters as for ssm_scan_fwd, except: p->y_dtype is the dtype of dy and of the per-step gradients dx, ddt, dz;
 *   p->segments is ignored (the backward always works in 64-step chunks).
 *   Inputs (device, as given to ssm_scan_fwd): x, dt, dt_bias, A, B, C, Dskip, z, h0;
 *     dy [batch][dim][seqlen] y_dtype;  dh_final [batch][dim][dstate] fp32 or NULL (= 0).
 *   Outputs (device, overwritten, never accumulated into):
 *     dx, ddt [batch][dim][seqlen] y_dtype (ddt is the gradient with respect to dt, through the softplus);
 *     dz [batch][dim][seqlen] y_dtype: required when z is given, must be NULL when it is not;
 *     dA [dim][dstate] fp32;  dB, dC [batch][dstate][seqlen] fp32 (summed over channels);
 *     dDskip [dim], ddt_bias [dim], dh0 [batch][dim][dstate] fp32, each optional (NULL = not computed).  dDskip and
 *     ddt_bias are the gradients at the given values, also when Dskip / dt_bias are NULL (i.e. at 0).
 *   workspace: device buffer of at least ssm_scan_bwd_workspace_bytes(p) bytes, 4-byte aligned.
 *   stream: hipStream_t or NULL.
 * Outputs must not overlap the inputs or each other.  Deterministic: every sum over channels, steps and batch runs in
 * a fixed order, so repeated calls give bit-identical results.
 */
ssm_status ssm_scan_bwd(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* Dskip, const void* z, const float* h0,
                        const void* dy, const float* dh_final, void* dx, void* ddt, float* dA, float* dB, float* dC,
                        float* dDskip, void* dz, float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Mamba-2 state space duality (SSD) layer: the selective recurrence with the state matrix reduced to a scalar times
 * the identity per head and a multi-head structure (alishangtian.com close reading, the paragraph on Mamba-2 and SSD;
 * docs.ifdog.com tutorial, "Mamba-2 与结构化对偶性", which names states of 128 or 256).  Channels are split into
 * nheads heads of headdim columns; head h uses group g = h / (nheads / ngroups) of B and C:
 *   Delta_t = softplus(dt[b,t,h] + dt_bias[h])   (or dt + dt_bias when dt_softplus == 0)
 *   S[p][n] <- exp(Delta_t A[h]) S[p][n] + phi_t B[b,t,g,n] x[b,t,h,p],
 *              phi_t = Delta_t (SSM_DISC_EULER_B) or expm1(Delta_t A[h]) / A[h] (SSM_DISC_ZOH; A == 0 gives Delta_t)
 *   y[b,t,h,p] = (sum_n C[b,t,g,n] S[p][n] + Dskip[h] x[b,t,h,p]) * silu(z[b,t,h,p])
 * The forward evaluates it in 64-step chunks as the masked quadratic (attention-like) form inside a chunk plus the
 * recurrence between chunks, on the bf16 matrix cores with fp32 accumulation and fp32 state.
 */
typedef struct {
  int64_t batch;       /* b >= 1 */
  int64_t seqlen;      /* L >= 1 (ignored by ssm_ssd_state_update) */
  int64_t nheads;      /* H >= 1, a multiple of ngroups */
  int64_t headdim;     /* P: must be 64 */
  int64_t ngroups;     /* G >= 1 */
  int64_t dstate;      /* N: 64, 128 or 256 */
  int32_t io_dtype;    /* must be SSM_BF16 (x, dt, B, C, z) */
  int32_t y_dtype;     /* SSM_BF16 or SSM_F32 */
  int32_t disc;        /* ssm_disc */
  int32_t dt_softplus; /* 1: Delta = softplus(dt + dt_bias); 0: Delta = dt + dt_bias */
  int32_t segments;    /* 0: the library picks how many L-segments run in parallel; k > 0 forces k (clamped to the
                          number of 64-step chunks); results agree within rounding either way */
} ssm_ssd_params;

/* Bytes of device workspace ssm_ssd_fwd needs (0 when it runs as one segment).  Pure host function. */
size_t ssm_ssd_fwd_workspace_bytes(const ssm_ssd_params* p);

/* Number of L-segments ssm_ssd_fwd uses for these parameters (>= 1), or 0 for invalid parameters. */
int ssm_ssd_fwd_plan_segments(const ssm_ssd_params* p);

/*
 * SSD forward over full sequences.  Layouts (row-major, heads inside time, as the pages' (batch, length, channels)):
 *   x, z [batch][seqlen][nheads][headdim] bf16 (z NULL = no gate);  dt [batch][seqlen][nheads] bf16;
 *   B, C [batch][seqlen][ngroups][dstate] bf16;  A, dt_bias, Dskip [nheads] fp32 (dt_bias / Dskip NULL = 0 / none);
 *   h0, h_final [batch][nheads][headdim][dstate] fp32 or NULL (h0 NULL = zeros; h_final may alias h0);
 *   y [batch][seqlen][nheads][headdim] y_dtype.
 * x, B, C, z, y, h0 and h_final must be 16-byte aligned.  workspace: device buffer of at least
 * ssm_ssd_fwd_workspace_bytes(p) bytes, 16-byte aligned (NULL if 0 are needed): with more than one segment a first
 * pass writes each segment's end state from a zero start there, and every segment starts from h0 carried through the
 * segments before it.  Errors as for ssm_scan_fwd, plus SSM_ERR_DTYPE for io_dtype != SSM_BF16,
 * SSM_ERR_UNSUPPORTED for headdim != 64, dstate not in {64, 128, 256} or negative segments, and SSM_ERR_SHAPE when
 * one batch element reaches 2^31 bytes (x or y counted at 4 bytes a value: seqlen * nheads * 64 * 4; B or C:
 * seqlen * ngroups * dstate * 2) or (seqlen + 128) steps of either reach 2^32 bytes (device offsets are 32-bit).
 */
ssm_status ssm_ssd_fwd(const ssm_ssd_params* p, const void* x, const void* dt, const float* dt_bias, const float* A,
                       const void* B, const void* C, const float* Dskip, const void* z, const float* h0, void* y,
                       float* h_final, void* workspace, size_t workspace_bytes, void* stream);

/* One SSD decode step: state [batch][nheads][headdim][dstate] fp32 (16-byte aligned) updated in place;
 * x, z, y [batch][nheads][headdim];  dt [batch][nheads];  B, C [batch][ngroups][dstate] (8-byte aligned). */
ssm_status ssm_ssd_state_update(const ssm_ssd_params* p, float* state, const void* x, const void* dt,
                                const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                                const void* z, void* y, void* stream);

/* Static description of a status code. */
const char* ssm_status_str(ssm_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* ssm_last_error(void);

/* SSM57_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

/* Number of L-segments ssm_scan_fwd would use for these parameters (>= 1), or 0 for invalid parameters. */
int ssm_scan_fwd_plan_segments(const ssm_scan_params* p);

#ifdef __cplusplus
}
#endif
#endif /* SSM57_SSM_SCAN_H */
