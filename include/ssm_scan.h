/*
 * ssm_scan.h - C ABI of the MI355X (gfx950) selective-scan library libssmscan.so.
 *
 * The library computes the Mamba selective state-space scan. For every batch
 * row b, channel d and step t:
 *
 *   delta_t = softplus(dt_raw[b,d,t] + dt_bias[d])              (beta = 1)
 *   h_t[n]  = exp(delta_t * A[d,n]) * h_{t-1}[n] + delta_t * B[b,t,n] * u[b,d,t]
 *   y_t     = sum_n C[b,t,n] * h_t[n] + D[d] * u[b,d,t]
 *   out     = y_t * silu(z[b,d,t])                               (y_t without z)
 *
 * with h_{-1} = h0 (zeros when absent) and, where reset[b,t] != 0, h_{t-1}
 * taken as zero before step t.
 *
 * Where each piece is defined (page titles; section names as on the pages):
 *  - the discrete recurrence h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t with
 *    Abar = exp(delta A), and the small-delta input matrix Bbar = delta B:
 *    "Illustrated Mamba state space model" (blog.luzhipeng.com), sections
 *    "Mathematical basis: structured SSM" and step 1 (discretisation);
 *  - delta = softplus(linear(x)) with B, C chosen per step: same page,
 *    "Mamba's innovation: the selection mechanism";
 *  - diagonal A, the per-step update state = A_t*state + B_t*u_t, the read-out
 *    with + D*u and the SiLU-gated block: "Mamba SSM core theory and
 *    Keras/TensorFlow implementation" (highthink.cn), SelectiveSSM layer;
 *  - the fused single kernel that loads parameters into on-chip memory,
 *    discretises and recurs there and writes back only the result:
 *    "Technical analysis: Mamba selective state spaces" (codechina.net),
 *    section 1 (hardware-aware algorithm) and 2.2 (kernel fusion);
 *  - document isolation by resetting the hidden state: same page, 3.2;
 *  - the single-token recurrent (RNN-style) inference step: "Reproducing
 *    Mamba's SSM core in Python" (mhpn.cn), section 3;
 *  - the causal depthwise convolution (width d_conv = 4) and SiLU that produce
 *    the scan input inside the Mamba block: "Illustrated Mamba state space
 *    model", the SSM module's conv1d (kernel_size = d_conv, padding d_conv-1,
 *    groups = d_model); "Mamba SSM core theory and Keras/TensorFlow
 *    implementation", block structure (causal Conv1D, then SiLU).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major in the layouts given below, each aligned to its element size.
 *    The library never allocates, frees or keeps them beyond the call.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream)
 *    and runs asynchronously; the call returns once it is enqueued.
 *  - Every argument check runs on the host before anything is enqueued, so a
 *    non-OK status means no device work was issued and no output was touched.
 *    Only SSM_ERR_HIP can follow a partial launch; ssm_last_error() then holds
 *    the HIP error text. Faults during execution surface at the caller's next
 *    synchronisation of the stream.
 *  - NaN/Inf inputs propagate by IEEE rules; they are not trapped.
 *  - Empty problems (B, D or L = 0) are valid: a pointer to an empty tensor
 *    may be NULL, nothing is scanned, and the outputs that still hold values
 *    get the empty sequence's: the state passes through it (h_last = h0, or
 *    0 without h0; conv_state_out = conv_state_in, or 0), its aggregate is
 *    the identity (P = 1, H = 0), empty sums are 0 (dA, dDskip, d_dt_bias,
 *    dconv_w, dconv_b over no (b, t); dBm, dCm over no channel), the adjoint passes through (dh0 = dh_last,
 *    or 0) and dconv_state_in is 0. No workspace is needed.
 *  - The library is re-entrant; its only global mutable state is the
 *    thread-local text returned by ssm_last_error().
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_VERSION 10900 /* major*10000 + minor*100 + patch */
#define SSM_MAX_DSTATE 256     /* largest supported N */

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL_POINTER = 1, /* a required pointer (or params itself) is NULL   */
  SSM_ERR_BAD_SHAPE = 2,    /* a size is < 0, N < 1, N > SSM_MAX_DSTATE,
                               L >= 2^27, or an element count overflows int64  */
  SSM_ERR_BAD_DTYPE = 3,    /* in_dtype / out_dtype is not an ssm_dtype         */
  SSM_ERR_MISALIGNED = 4,   /* a pointer is not aligned to its element size    */
  SSM_ERR_UNSUPPORTED = 5,  /* a valid request the library does not implement */
  SSM_ERR_WORKSPACE = 6,    /* workspace smaller than ssm_scan_workspace_size() */
  SSM_ERR_ALIAS = 7,        /* an output overlaps an input, another output or
                               the workspace                                   */
  SSM_ERR_HIP = 8           /* the HIP runtime refused a call; see ssm_last_error */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* How the input matrix is discretised (the `discretization` field):
 *  SSM_DISC_DELTA_B  Bbar = delta * B, the small-delta form ("Illustrated Mamba
 *                    state space model", step 1; "Mamba SSM core theory and
 *                    Keras/TensorFlow implementation", scan step). Default.
 *  SSM_DISC_ZOH      Bbar = (exp(delta A) - 1) / A * B, the exact zero-order hold
 *                    of the diagonal continuous system ("Illustrated Mamba state
 *                    space model", "Mathematical basis: structured SSM"; also
 *                    "Reproducing Mamba's SSM core in Python", section 1); delta * B where A = 0.
 * Abar = exp(delta A) in both. Other values return SSM_ERR_UNSUPPORTED. */
typedef enum { SSM_DISC_DELTA_B = 0, SSM_DISC_ZOH = 1 } ssm_discretization;

/* Kind of the diagonal state (the `state_kind` field):
 *  SSM_STATE_REAL     real A, B, C and h, as above. Default.
 *  SSM_STATE_COMPLEX  the complex-diagonal variant whose initialisation the
 *                     pages give as A = -1/2 + i n (S4D-Lin) and whose complex
 *                     state keeps phase information ("Technical analysis: Mamba
 *                     selective state spaces", sections 4.1 and 5.3). A, B, C,
 *                     h0, h_last and the decode state h are complex, stored as
 *                     interleaved (re, im) pairs: every such tensor gains a
 *                     trailing dimension of 2 (A (D,N,2) float32, Bm and Cm
 *                     (B,L,N,2) or (B,N,2) in in_dtype, states (B,D,N,2) float32).
 *                     delta, u, z and out stay real; the recurrence is
 *                       h_t[n] = exp(delta_t A[d,n]) h_{t-1}[n] + delta_t B[b,t,n] u
 *                       y_t    = Re(sum_n C[b,t,n] h_t[n]) + D[d] u
 *                     (with SSM_DISC_ZOH the input coefficient is the complex
 *                     (exp(delta A) - 1) / A in place of delta), with the same
 *                     gate, resets and optional conv stage. It is supported in
 *                     ssm_scan_fwd (whose workspace then holds complex
 *                     aggregates; ask ssm_scan_workspace_size with state_kind
 *                     set), ssm_scan_aggregate, ssm_state_update and
 *                     ssm_scan_bwd.
 * Other values return SSM_ERR_UNSUPPORTED. */
typedef enum { SSM_STATE_REAL = 0, SSM_STATE_COMPLEX = 1 } ssm_state_kind;

/*
 * Full-sequence scan (prefill / training forward).
 *
 *   batch, dim, seqlen, dstate : B, D, L, N;  B, D >= 0, 0 <= L < 2^27, 1 <= N <= 256
 *   in_dtype  : element type of u, dt_raw, z, Bm, Cm (SSM_F32 or SSM_BF16)
 *   out_dtype : element type of out (SSM_F32 or SSM_BF16)
 *   u        (B,D,L)  required; the SSM input x (L contiguous)
 *   dt_raw   (B,D,L)  required; pre-softplus step size
 *   dt_bias  (D)      float32, NULL => 0
 *   A        (D,N)    float32, required; the diagonal of the state matrix.
 *                     Any real value is accepted; stable models have A <= 0.
 *   Bm, Cm   (B,L,N)  required; input and output matrices per step (N contiguous)
 *   Dskip    (D)      float32, NULL => no skip term
 *   z        (B,D,L)  NULL => no gate (out = y)
 *   reset    (B,L)    uint8, NULL => none; nonzero at t clears the state before step t
 *   h0       (B,D,N)  float32, NULL => zero initial state
 *   out      (B,D,L)  required; written once per element; must not overlap inputs
 *   h_last   (B,D,N)  float32, NULL => not written; the state after step L-1
 *   workspace, workspace_bytes : scratch for scans that split the sequence
 *                     across workgroups; at least ssm_scan_workspace_size()
 *                     bytes (may be NULL when that size is 0). Its contents on
 *                     entry are ignored; callers may reuse it between calls on
 *                     the same stream.
 *   num_segments : 0 = the library chooses how many pieces to split L into;
 *                  k >= 1 asks for k pieces (clamped to what L allows).
 *
 * Optional input stage (conv_w != NULL): u holds the input x of a causal
 * depthwise convolution, and the scan runs on
 *   u'_t = silu(conv_b[d] + sum_{k<K} conv_w[d,k] * x_{t-K+1+k}),  K = conv_width
 * in place of u everywhere (delta*u' and D*u'). The convolution does not look
 * across a reset: inputs before the start of the current document count as 0.
 *   conv_w         (D,K)   float32; 1 <= conv_width <= 4
 *   conv_b         (D)     float32, NULL => 0
 *   conv_state_in  (B,D,K-1) float32, NULL => zeros; x_{-K+1} .. x_{-1}, oldest first
 *   conv_state_out (B,D,K-1) float32, NULL => not written; the last K-1 inputs
 *                  of the sequence (zeros for those hidden by a later reset),
 *                  ready to be the next call's conv_state_in
 * conv_width is ignored when conv_w is NULL.
 */
typedef struct {
  int64_t batch, dim, seqlen, dstate;
  int32_t in_dtype, out_dtype;
  const void* u;
  const void* dt_raw;
  const float* dt_bias;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const uint8_t* reset;
  const float* h0;
  void* out;
  float* h_last;
  void* workspace;
  size_t workspace_bytes;
  int32_t num_segments;
  int32_t discretization; /* ssm_discretization */
  const float* conv_w;
  const float* conv_b;
  const float* conv_state_in;
  float* conv_state_out;
  int32_t conv_width;
  int32_t state_kind; /* ssm_state_kind */
} ssm_scan_params;

/* Bytes of workspace ssm_scan_fwd needs for these parameters (0 when the scan
 * does not split the sequence). Only the sizes, dtypes, num_segments and
 * state_kind of `p` are read. */
ssm_status ssm_scan_workspace_size(const ssm_scan_params* p, size_t* bytes);

/* Enqueue the scan described by `p` on `hip_stream`. */
ssm_status ssm_scan_fwd(const ssm_scan_params* p, void* hip_stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same scan
 * as ssm_scan_fwd, with the same arguments, results and errors, except that
 * workspace and workspace_bytes are ignored: a scan that splits the sequence
 * keeps its pieces' aggregates in scratch memory the library owns, a fixed
 * array of SSM_NOALLOC_SCRATCH_BYTES on every device it runs on (held until
 * the process ends; its address is looked up on the first call per device).
 * The call allocates and frees nothing. Nothing in the scratch needs to start
 * at zero: every piece's aggregate is written before it is read.
 *   - A split whose aggregates need more than SSM_NOALLOC_SCRATCH_BYTES
 *     (ssm_scan_workspace_size() reports the need) returns SSM_ERR_WORKSPACE
 *     before any launch.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents: calls that may overlap on one GPU (different streams,
 *     no ordering between them) race and must be serialised by the caller.
 *   - The scratch address lookup can fail with SSM_ERR_HIP.
 */
#define SSM_NOALLOC_SCRATCH_BYTES (16u << 20)
ssm_status ssm_scan_fwd_noalloc(const ssm_scan_params* p, void* hip_stream);

/*
 * The same forward computed as a chunked two-level associative scan, the
 * parallel form of the recurrence ("Technical analysis: Mamba selective state
 * spaces", 2.2, the parallel scan in place of the serial recursion): one wave
 * per (b, d), one step per lane of a 64-step chunk; per state the affine
 * pairs (exp(delta_t A[d,n]), delta_t B[b,t,n] u_t) are composed by a
 * wavefront scan with DPP lane moves (six levels), and the state after each
 * chunk carries into the next. It exists to measure that design against
 * ssm_scan_fwd's sequential-in-lane kernels, which are faster on gfx950; the
 * results agree with ssm_scan_fwd's within rounding (the products of the decays
 * are formed in a different order).
 *   p : as for ssm_scan_fwd, restricted to dstate = 16, state_kind
 *       SSM_STATE_REAL, discretization SSM_DISC_DELTA_B and no conv stage
 *       (others return SSM_ERR_UNSUPPORTED before any launch), with Bm and
 *       Cm aligned to 16 bytes (else SSM_ERR_MISALIGNED). The sequence is
 *       never split: workspace, workspace_bytes and num_segments are
 *       ignored, and nothing is allocated. Other errors as for ssm_scan_fwd.
 */
ssm_status ssm_scan_fwd_wavefront(const ssm_scan_params* p, void* hip_stream);

/*
 * Affine aggregate of a whole sequence, for scanning one sequence in shards
 * (the pages advise processing extremely long sequences in chunks: "Technical
 * analysis: Mamba selective state spaces", section 7), for instance one shard
 * per device. For the inputs of ssm_scan_fwd the sequence maps the state h
 * entering it to P h + H, per (b, d, n), with
 *   P = prod_t exp(delta_t A[d,n])   (0 when a reset lies in the sequence)
 *   H = the state after the sequence from a zero state (same input
 *       coefficient, resets and conv stage as the forward).
 * Scanning consecutive shards s = 0, 1, ...: each computes (P_s, H_s); the
 * state entering shard s is h_s = P_{s-1} h_{s-1} + H_{s-1} (h_0: the
 * sequence's h0); ssm_scan_fwd of shard s with h0 = h_s gives its outputs.
 * With the conv stage, a shard's conv_state_in is the preceding shard's last
 * K-1 inputs.
 *   p    : read as for ssm_scan_fwd: batch .. dstate, in_dtype, u, dt_raw,
 *          dt_bias, A, Bm, reset, conv_w, conv_b, conv_state_in, conv_width,
 *          discretization, state_kind, num_segments, workspace; out_dtype,
 *          z, Cm, Dskip, h0, out, h_last and conv_state_out are not read.
 *   P, H : (B,D,N) float32 outputs ((B,D,N,2) with the complex state),
 *          4-byte aligned, overlapping neither the inputs, each other nor the
 *          workspace. Errors as for ssm_scan_fwd, all detected before any launch.
 */
ssm_status ssm_scan_aggregate(const ssm_scan_params* p, float* P, float* H, void* hip_stream);

/* Bytes of workspace ssm_scan_aggregate needs (0 unless the library splits
 * the sequence into pieces); sizes, dtypes, flags and num_segments are read. */
ssm_status ssm_scan_aggregate_workspace_size(const ssm_scan_params* p, size_t* bytes);

/*
 * Single-token decode step: one application of the recurrence to a stored
 * state, in place.
 *
 *   batch, dim, dstate : B, D, N;  B, D >= 0, 1 <= N <= 256
 *   h        (B,D,N)  float32, required; read as h_{t-1}, overwritten with h_t.
 *                     To start a new sequence the caller zeroes that row.
 *   u, dt_raw (B,D)   required; z (B,D) NULL => no gate
 *   dt_bias  (D), Dskip (D) float32, NULL => 0 / no skip term; A (D,N) float32
 *   Bm, Cm   (B,N)    required
 *   out      (B,D)    required; must not overlap h or any input
 *   conv_w   (D,K)    float32, NULL => no conv stage; with it, u is this step's
 *                     conv input and the step input is
 *                     silu(conv_b + sum_k conv_w[d,k] * window[k]) over the window
 *                     (conv_state[b,d,0 .. K-2], u), K = conv_width in [1, 4]
 *   conv_b   (D)      float32, NULL => 0
 *   conv_state (B,D,K-1) float32, required with conv_w when K > 1: the previous
 *                     K-1 inputs, oldest first; shifted in place by one input.
 *                     Must not overlap h, out or any input.
 */
typedef struct {
  int64_t batch, dim, dstate;
  int32_t in_dtype, out_dtype;
  float* h;
  const void* u;
  const void* dt_raw;
  const void* z;
  const float* dt_bias;
  const float* A;
  const float* Dskip;
  const void* Bm;
  const void* Cm;
  void* out;
  float* conv_state;
  const float* conv_w;
  const float* conv_b;
  int32_t conv_width;
  int32_t discretization; /* ssm_discretization */
  int32_t state_kind;     /* ssm_state_kind */
  int32_t reserved1;      /* set to 0 */
} ssm_update_params;

/* Enqueue the decode step described by `p` on `hip_stream`. */
ssm_status ssm_state_update(const ssm_update_params* p, void* hip_stream);

/*
 * Backward pass of the full-sequence scan: the gradients of
 *
 *   loss = sum_{b,d,t} dout[b,d,t] * out[b,d,t] + sum_{b,d,n} dh_last[b,d,n] * h_last[b,d,n]
 *
 * with respect to every input of ssm_scan_fwd, for the same inputs. The
 * forward keeps no intermediate states; the backward recomputes them
 * ("Technical analysis: Mamba selective state spaces", section 2.2, item 3:
 * gradient recomputation). The gradients are the chain rule through the
 * recurrence above, run in reverse time:
 *
 *   g_t     = adjoint of h_t = a_{t+1} g_{t+1} + dy_t C_t,  dy_t = dout_t silu(z_t)
 *   dB[b,t,n] = sum_d g_t[n] delta_t u_t          dC[b,t,n] = sum_d dy_t h_t[n]
 *   dA[d,n]   = sum_{b,t} g_t[n] a_t[n] h_{t-1}[n] delta_t
 *   du_t      = dy_t D + delta_t sum_n g_t[n] B_t[n]
 *   d dt_raw_t = (sum_n g_t[n] (A[n] a_t[n] h_{t-1}[n] + B_t[n] u_t)) sigmoid(dt_raw_t + dt_bias)
 *   dz_t      = dout_t y_t silu'(z_t);  dD = sum dy u;  d dt_bias = sum d dt_raw
 *   dh0       = a_0 g_0
 *
 * with a_t = exp(delta_t A) (0 where reset[b,t] clears the state) and h_{-1} = h0.
 *
 *   batch .. h0 : as in ssm_scan_params (the forward's inputs, unchanged)
 *   in_dtype   : element type of u, dt_raw, z, Bm, Cm and dout
 *   grad_dtype : element type of du, d_dt_raw and dz (SSM_F32 or SSM_BF16)
 *   dout     (B,D,L)  required; gradient of the loss with respect to out
 *   dh_last  (B,D,N)  float32, NULL => 0
 *   du, d_dt_raw (B,D,L) required outputs
 *   dz       (B,D,L)  required when z is given, must be NULL otherwise
 *   dA       (D,N)    float32, required output
 *   dBm, dCm (B,L,N)  float32, required outputs
 *   dDskip, d_dt_bias (D) float32 outputs, NULL => not written. They are the
 *                     gradients with respect to D and dt_bias whether or not
 *                     those inputs are given (an absent input acts as 0).
 *   dh0      (B,D,N)  float32 output, NULL => not written
 *   workspace, workspace_bytes : at least ssm_scan_bwd_workspace_size() bytes
 *                     (0 only for an empty problem); contents on entry ignored.
 * Conv input stage (conv_w != NULL, as in ssm_scan_params): u is the conv
 * input x; du is the gradient of x, and
 *   conv_w, conv_b, conv_state_in, conv_width : the forward's conv arguments
 *   dconv_w (D,K), dconv_b (D), dconv_state_in (B,D,K-1) float32 outputs,
 *                     NULL => not written
 * Complex state (state_kind = SSM_STATE_COMPLEX):
 * A, Bm, Cm, h0, dh_last and dA, dBm, dCm, dh0 gain a trailing (re, im)
 * dimension of 2, as in the forward. The loss's h_last term is
 * sum (Re dh_last Re h_last + Im dh_last Im h_last), and the gradient of a
 * complex input x is stored as (dL/dRe x, dL/dIm x). With G_t that form of
 * the adjoint of h_t, the formulas above become
 *   G_t = conj(a_{t+1}) G_{t+1} + dy_t conj(C_t),   dC = sum_d dy_t conj(h_t),
 *   dB = sum_d delta_t u_t G_t,   dA = sum_{b,t} delta_t G_t conj(a_t h_{t-1}),
 *   du_t = dy_t D + delta_t Re sum_n conj(G_t) B_t,
 *   d dt_raw_t = Re(sum_n conj(G_t) (A a_t h_{t-1} + B_t u_t)) sigmoid(..),
 *   dh0 = conj(a_0) G_0,
 * and y_t in dz_t is the real read-out Re sum_n C_t h_t + D u_t. With
 * SSM_DISC_ZOH the input coefficient delta becomes q = (e^{delta A} - 1)/A:
 *   dB = sum_d u_t conj(q_t) G_t,   du_t = dy_t D + Re sum_n conj(G_t) q_t B_t,
 *   d dt_raw_t gains Re sum_n conj(G_t) a_t B_t u_t in place of the B_t u_t
 *   term (d q/d delta = a), and dA gains u_t G_t conj(dq/dA B_t),
 *   dq/dA = (delta a_t - q_t)/A.
 * Outputs must not overlap each other, the inputs or the workspace. Shared
 * gradients (dA, dBm, dCm, dDskip, d_dt_bias, dconv_w, dconv_b) are sums in a
 * fixed order, so repeated calls give identical bits.
 */
typedef struct {
  int64_t batch, dim, seqlen, dstate;
  int32_t in_dtype, grad_dtype;
  const void* u;
  const void* dt_raw;
  const float* dt_bias;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const uint8_t* reset;
  const float* h0;
  const void* dout;
  const float* dh_last;
  void* du;
  void* d_dt_raw;
  void* dz;
  float* dA;
  float* dBm;
  float* dCm;
  float* dDskip;
  float* d_dt_bias;
  float* dh0;
  void* workspace;
  size_t workspace_bytes;
  const float* conv_w;
  const float* conv_b;
  const float* conv_state_in;
  float* dconv_w;
  float* dconv_b;
  float* dconv_state_in;
  int32_t conv_width;
  int32_t discretization; /* ssm_discretization */
  int32_t state_kind;     /* ssm_state_kind */
  int32_t reserved1;      /* set to 0 */
} ssm_scan_bwd_params;

/* Bytes of workspace ssm_scan_bwd needs (only sizes and dtypes of `p` are read). */
ssm_status ssm_scan_bwd_workspace_size(const ssm_scan_bwd_params* p, size_t* bytes);

/* Enqueue the backward pass described by `p` on `hip_stream`. */
ssm_status ssm_scan_bwd(const ssm_scan_bwd_params* p, void* hip_stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* ssm_status_string(int32_t status);

/* Detail of the last non-OK status returned on this thread (static storage,
 * valid until the next library call on this thread). */
const char* ssm_last_error(void);

/* SSM_SCAN_VERSION of the loaded library. */
int32_t ssm_version(void);

/* sizeof of the parameter structs as compiled into the library:
 * which = 0 -> ssm_scan_params, 1 -> ssm_update_params,
 * 2 -> ssm_scan_bwd_params; 0 for anything else.
 * Bindings compare these with their own layouts at load time. */
size_t ssm_abi_struct_size(int32_t which);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
