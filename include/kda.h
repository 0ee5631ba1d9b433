/*
 * kda.h -- C ABI of libkda, the Kimi Delta Attention (KDA) token mixer for
 * AMD Instinct MI355X (gfx950).
 *
 * The mixer (the token mixer of 69 of the 93 layers of Kimi-K3, with a state of
 * fixed size per head: "Kimi-K3 model atlas -- self.layers"; geometry from the
 * released config's linear_attn_config: num_heads 96, head_dim 128,
 * short_conv_kernel_size 4, full-rank gate) computes, per sequence b and head h:
 *
 *   1. causal depthwise conv over time, kernel K = conv_k (no bias), then SiLU,
 *      on q, k and v separately:  y[t,c] = SiLU( sum_tau w[c,tau] x[t-(K-1)+tau, c] )
 *      (filters stored per channel as [H*D, 1, K] float32: "MaxText PR 5548",
 *      review item 2; the last tap multiplies the current token);
 *   2. L2 normalisation of q and k over the head's D channels:
 *      x / sqrt(sum x^2 + l2_eps)   (l2_eps defaults to 1e-6, the eps the pages
 *      fix for KimiRMSNorm: "Kimi-K3 atlas -- MoE input (decode)");
 *   3. the channel-wise gated delta rule with a D x D float32 state,
 *      S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,
 *      o_t = scale * S_t^T q_t   (decay per key channel; the output reads S_t).
 *
 * Optional stages around it, each off unless its pointers are given:
 *   - decay and write strength from raw projections: g = -exp(A_log[h]) *
 *     softplus(f + dt_bias[h*D + c]) with f the gate projection, evaluated in
 *     float32 (A_log [num_heads] and dt_bias [H*D] are kept in float32 because
 *     bf16 copies drift the decay over long contexts: "MaxText PR 5548", review
 *     item 2; the softplus form is this library's reading, the pages give only
 *     the parameters), and beta = sigmoid(b) with flag KDA_FLAG_BETA_LOGITS;
 *   - the output RMSNorm of each head with the layer's o_norm gain ([head_dim],
 *     float32: "MaxText PR 5548", review item 2; the norm as KimiRMSNorm:
 *     "Kimi-K3 atlas -- MoE input (decode)"), then the sigmoid output gate of
 *     the g_proj output (the gate form of "MaxText PR 5543", What, item 1):
 *     o <- o / sqrt(mean_c o_c^2 + o_norm_eps) * o_norm_w * sigmoid(o_gate).
 *     The gate_lower_bound of the released config is not applied (the pages do
 *     not say how it enters).
 *
 * Conventions for every entry point
 *   - Ownership: the caller owns every buffer.  The library never allocates or
 *     frees device memory and keeps no global mutable state (reentrant; any
 *     number of streams).  Scratch memory is the caller's workspace -- except
 *     for kda_prefill_static, whose workspace is a static array per GPU.
 *   - Pointers named "device" are device (HBM) addresses; they must be 16-byte
 *     aligned.  Argument structs themselves live in host memory.
 *   - Asynchrony: compute entry points enqueue kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and return.  Launch
 *     failures are reported as KDA_ERR_HIP; faults during execution surface at
 *     the caller's next synchronisation.
 *   - All-or-nothing: every argument is validated on the host before anything is
 *     enqueued; on any error nothing is launched and outputs are untouched.
 *     Validation never calls into the HIP runtime and never reads device memory.
 *   - Unsupported modes return KDA_ERR_UNSUPPORTED instead of computing a wrong
 *     result (D outside {16,32,64,128}, conv_k outside {0,4}, chunk outside
 *     {16,32,64}, fp32 I/O with D = 128 and chunk = 64).  Packed variable-length
 *     sequences are supported by kda_prefill (cu_seqlens; the layers the pages
 *     describe reject packing because their KDA would let state flow across
 *     segment boundaries: "MaxText PR 5550").
 *   - Device values are not checked: g must be finite and <= 0 (any finite value
 *     when it holds a raw projection), inputs finite.
 *
 * Layouts (row-major, innermost last; dtype = `io` unless stated):
 *   q, k, v, g, o   [B][T][H][D]        (decode: [B][H][D])
 *   beta            [B][T][H]           (decode: [B][H])
 *   conv_w          [3][H*D][conv_k]    float32, filters of q, k, v in that order
 *   conv state      [B][3][conv_k-1][H*D]  raw (pre-conv) inputs, oldest first
 *   S0, S_T, S      [B][H][D][D]        float32, row = key channel, col = value channel
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL (or conv_w given with conv_k = 0) */
  KDA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or overflows */
  KDA_ERR_DTYPE = 3,       /* io is not a kda_dtype */
  KDA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  KDA_ERR_ALIAS = 5,       /* an output overlaps an input it may not overlap */
  KDA_ERR_UNSUPPORTED = 6, /* valid request outside what this build implements */
  KDA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than the query says */
  KDA_ERR_HIP = 8,         /* the HIP runtime refused a launch */
  KDA_ERR_VALUE = 9,       /* a scalar argument is out of range (eps, scale, flags, stage) */
  KDA_ERR_SCRATCH = 10     /* kda_prefill_static: the request needs more than the static scratch */
} kda_status;

typedef enum kda_dtype {
  KDA_BF16 = 0, /* bfloat16 I/O, bf16 matrix-core products with float32 accumulation */
  KDA_FP32 = 1  /* float32 I/O and float32 arithmetic throughout */
} kda_dtype;

/* flags */
#define KDA_FLAG_L2NORM_QK (1u << 0) /* apply step 2 (the released model does) */
#define KDA_FLAG_BETA_LOGITS (1u << 1) /* beta holds logits b; the write strength is sigmoid(b) */
#define KDA_FLAGS_DEFAULT KDA_FLAG_L2NORM_QK

/* ------------------------------------------------------------------ prefill */
/* Whole-sequence forward of the mixer for B equal-length sequences.
 *
 * The recurrence is evaluated in chunks of `chunk` tokens: per chunk a cumulative
 * log-decay, the masked intra-chunk key products, a unit-lower-triangular solve
 * (the WY/UT form of the delta rule), then a serial walk over chunks that carries
 * the D x D state.  The chunk length changes rounding only, not the result.
 */
typedef struct kda_prefill_args {
  int32_t B, T, H, D;   /* batch, tokens (>= 0), heads, head_dim (keys and values) */
  int32_t chunk;        /* 16 | 32 | 64 (64 recommended for D = 128) */
  int32_t conv_k;       /* 4, or 0 = inputs are already convolved + activated */
  uint32_t flags;       /* KDA_FLAG_* */
  float l2_eps;         /* >= 0, finite; 1e-6 in the released model */
  float scale;          /* finite; output scale (1.0 in the released model) */
  int32_t io;           /* kda_dtype of q, k, v, g, beta, o, conv states */
  const void* q;        /* device [B][T][H][D] raw queries */
  const void* k;        /* device [B][T][H][D] raw keys */
  const void* v;        /* device [B][T][H][D] raw values */
  const void* g;        /* device [B][T][H][D] log-decay per key channel (finite, <= 0) */
  const void* beta;     /* device [B][T][H] write strength */
  const float* conv_w;  /* device [3][H*D][conv_k] float32; NULL iff conv_k == 0 */
  const void* conv_state_in;  /* device [B][3][conv_k-1][H*D] or NULL (= zeros) */
  const float* S0;      /* device [B][H][D][D] initial state or NULL (= zeros) */
  void* o;              /* device [B][T][H][D] output; may not overlap any input */
  float* S_T;           /* device [B][H][D][D] final state; may equal S0 (in place) */
  void* conv_state_out; /* device [B][3][conv_k-1][H*D] or NULL; may equal conv_state_in */
  /* optional stages (NULL = off) */
  const float* A_log;   /* device [H] float32; given iff dt_bias is.  Then g holds the raw
                           gate projection f and the decay is -exp(A_log[h]) softplus(f + dt_bias) */
  const float* dt_bias; /* device [H*D] float32 */
  const float* o_norm_w;/* device [D] float32 gain of the output RMSNorm (shared by the heads) */
  float o_norm_eps;     /* >= 0, finite; read only with o_norm_w (1e-6 in the released model) */
  const void* o_gate;   /* device [B][T][H][D] gate pre-activation: o <- o * sigmoid(o_gate),
                           after the norm if both are given */
  /* packed sequences (NULL = B equal-length sequences) */
  const int32_t* cu_seqlens; /* device [n_seqs + 1] token offsets, 0 = cu[0] <= cu[1] <= ...
                                <= cu[n_seqs] = T; requires B = 1.  Sequence i is tokens
                                [cu[i], cu[i+1]) with its own conv history and initial state:
                                S0, S_T are [n_seqs][H][D][D] and the conv states
                                [n_seqs][3][conv_k-1][H*D].  Offsets are read on the device
                                and clamped (running maximum, within [0, T]): malformed ones
                                give wrong sequences but no access outside the buffers, and
                                tokens outside every sequence leave o undefined. */
  int32_t n_seqs;       /* >= 1 with cu_seqlens; must be 0 without */
} kda_prefill_args;

/* Host-only check of every argument; returns the first error found. */
kda_status kda_validate_prefill(const kda_prefill_args* a);

/* Bytes of device workspace kda_prefill needs for these sizes (0 if invalid). */
size_t kda_prefill_workspace_bytes(const kda_prefill_args* a);

/* Enqueue the whole forward on `stream`.  ws: device workspace of at least
 * kda_prefill_workspace_bytes(a) bytes, 256-byte aligned, not shared with a call
 * that may run concurrently.  T == 0 copies S0 (or zeros) to S_T and the conv
 * state through. */
kda_status kda_prefill(const kda_prefill_args* a, void* ws, size_t ws_bytes, void* stream);

/* The stages kda_prefill enqueues, one at a time, for profiling:
 *   0 = chunk preparation (conv + SiLU + L2, cumulative decay, intra-chunk
 *       products, triangular solve, and the activation of raw projections;
 *       writes the workspace),
 *   1 = state walk over chunks with the output (reads the workspace; writes o, S_T;
 *       applies the output norm and gate itself when one workgroup holds a
 *       head's whole output row),
 *   2 = conv-state hand-over (writes conv_state_out),
 *   3 = the output norm and gate as a separate in-place pass over o, when stage 1
 *       did not apply them (nothing otherwise).
 *   4 = stages 1 and 2 in one launch: the state walk's first value block per head
 *       also writes the conv-state hand-over (the preparation has read the
 *       previous state by then, so the new one may overwrite it).
 * Running 0, 1, 2, 3 or 0, 4, 3 in order on one stream gives exactly kda_prefill's
 * results (T > 0); kda_prefill itself enqueues 0, 4, 3. */
#define KDA_STAGE_PREP 0
#define KDA_STAGE_STATE 1
#define KDA_STAGE_CONV_TAIL 2
#define KDA_STAGE_OUTPUT 3
#define KDA_STAGE_STATE_TAIL 4
kda_status kda_prefill_stage(const kda_prefill_args* a, void* ws, size_t ws_bytes, int stage,
                             void* stream);

/* Host-only: the number of segments the state walk of kda_prefill(a) is split
 * into, 1 when it is not split, 0 when the arguments are invalid.  The state
 * after a run of tokens is affine in the state before it (S_end = M S_start + N,
 * M acting on the key index: each step of the update in item 3 above maps S
 * linearly, by (I - beta k k^T) Diag(exp(g)), and adds beta k v^T).
 * When the walks of a call are too few to fill the GPU while each is a long
 * chain of chunk steps (few sequence-heads, long T: a tensor-parallel share of
 * heads at long context), every (sequence, head) is cut into segments: each
 * segment's N and M are walked in parallel, the start states composed in order,
 * then each segment walked with its outputs from its start.  Only B equal-length
 * sequences with T > 0 split, and never a walk that applies the output stage
 * itself.  The results agree with the unsplit walk's to rounding (the same sums
 * in another order); the workspace includes the segments' maps and start states
 * (4 nseg - 3 float32 D x D matrices per (sequence, head)).  kda_prefill_backward
 * splits both of its walks the same way: the reverse walk is affine in the
 * gradient of the end state with the transposed maps M^T of the forward. */
int kda_prefill_walk_segments(const kda_prefill_args* a);

/* The affine state map of a prefill call, for splitting one sequence over
 * devices (each device its contiguous share of the tokens): per (sequence, head),
 * the state after the call's tokens is S_T = M S_start + N for any state
 * S_start before them, where N is the state reached from zero and M
 * (D x D, acting on the key index) the product of the steps' linear parts
 * (I - beta k k^T) Diag(exp(g)) (see kda_prefill_walk_segments).  A device
 * holding the later tokens computes its (M, N) without knowing S_start; once
 * the shares before it have handed over their maps (S_start = M' S' + N',
 * composed in order; M and N are 64 KB each per head in float32 at D = 128),
 * it runs stages 1 to 3 from S0 = S_start on the same workspace.
 *   - Call after kda_prefill_stage(a, ws, ws_bytes, KDA_STAGE_PREP, stream) on
 *     the same stream with the same arguments and workspace: the map is formed
 *     from the chunk records that stage wrote.  ws_bytes must be at least
 *     kda_prefill_state_map_workspace_bytes(a) (at least the prefill's); a later
 *     stage 1 on the same workspace is unaffected.  a->S0 is not read.
 *   - M, N: device [B][H][D][D] float32, row = key channel of S_T; written.  They
 *     may not overlap each other, any buffer of a, or the workspace.
 *   - B equal-length sequences only (packed: KDA_ERR_UNSUPPORTED).  T = 0 gives
 *     M = I, N = 0 (no workspace needed).
 *   - The maps of the call's segments (cut as the split walk cuts) are walked in
 *     parallel and composed in float32; rounding as in the walk itself. */
size_t kda_prefill_state_map_workspace_bytes(const kda_prefill_args* a);
kda_status kda_prefill_state_map(const kda_prefill_args* a, void* ws, size_t ws_bytes, float* M,
                                 float* N, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: kda_prefill
 * with its workspace taken from a static device array of
 * KDA_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on (one
 * array per GPU, from the first call there until the process ends).  It
 * allocates nothing and takes no workspace argument; the caller still provides
 * every input and output.  Same arguments, rules and results as kda_prefill.
 *   - When the whole-sequence workspace (kda_prefill_workspace_bytes) fits the
 *     array, the call runs exactly as kda_prefill.  Otherwise B equal-length
 *     sequences are processed in time slices of as many chunks per (sequence,
 *     head) as fit, the state handed from slice to slice through S_T; the
 *     results are the same bit for bit, except where kda_prefill would split
 *     its state walk (kda_prefill_walk_segments > 1: slices walk unsplit, so
 *     the two agree to rounding).  Packed sequences that do not fit, and
 *     any request of which not even one chunk per (sequence, head) fits (more
 *     than about 1,800 sequence-heads at D = 128, chunk 64, bf16), return
 *     KDA_ERR_SCRATCH before anything is enqueued.
 *   - The stream must belong to the current device (hipSetDevice).
 *   - Every call on one GPU shares that GPU's array: calls that may overlap on
 *     one GPU (other streams, other host threads) race and must be serialised
 *     by the caller.  Stream order serialises calls on one stream. */
#define KDA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
kda_status kda_prefill_static(const kda_prefill_args* a, void* stream);

/* ---------------------------------------------------------------- conv_norm */
/* Step 1 and 2 alone: writes the convolved, activated (and for q, k normalised)
 * inputs, as the recurrence consumes them.  Same layouts and rules as prefill. */
typedef struct kda_conv_norm_args {
  int32_t B, T, H, D;
  int32_t conv_k;       /* 4 (0 is rejected: nothing to do) */
  uint32_t flags;
  float l2_eps;
  int32_t io;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;        /* device [3][H*D][conv_k] */
  const void* conv_state_in;  /* device or NULL */
  void* q_out;                /* device [B][T][H][D] */
  void* k_out;
  void* v_out;
  void* conv_state_out;       /* device or NULL; may equal conv_state_in */
} kda_conv_norm_args;

kda_status kda_validate_conv_norm(const kda_conv_norm_args* a);
kda_status kda_conv_norm(const kda_conv_norm_args* a, void* stream);

/* ------------------------------------------------------------------- decode */
/* One autoregressive step for B sequences (T = 1): conv ring shift, SiLU, L2,
 * then the state update and output, the state read and written once, in place.
 * This is the cached-state decode that MaxText's KDA lacks ("MaxText PR 5550",
 * Known limitations). */
typedef struct kda_decode_args {
  int32_t B, H, D;
  int32_t conv_k;       /* 4 or 0 */
  uint32_t flags;
  float l2_eps;
  float scale;
  int32_t io;
  const void* q;        /* device [B][H][D] raw */
  const void* k;
  const void* v;
  const void* g;        /* device [B][H][D] log-decay (finite, <= 0) */
  const void* beta;     /* device [B][H] */
  const float* conv_w;  /* device [3][H*D][conv_k]; NULL iff conv_k == 0 */
  void* conv_state;     /* device [B][3][conv_k-1][H*D] in/out; required iff conv_k > 0 */
  float* S;             /* device [B][H][D][D] in/out, updated in place */
  void* o;              /* device [B][H][D]; may not overlap any input */
  /* optional stages, as in kda_prefill_args */
  const float* A_log;   /* device [H] float32; given iff dt_bias is (g then holds f) */
  const float* dt_bias; /* device [H*D] float32 */
  const float* o_norm_w;/* device [D] float32 or NULL */
  float o_norm_eps;
  const void* o_gate;   /* device [B][H][D] or NULL */
} kda_decode_args;

kda_status kda_validate_decode(const kda_decode_args* a);
kda_status kda_decode_step(const kda_decode_args* a, void* stream);

/* --------------------------------------------------------------- backward */
/* Gradients of the prefill: with do and dS_T the gradients of a loss with
 * respect to o and S_T, the gradients of L = <o, do> + <S_T, dS_T> with respect
 * to the raw q, k, v, g, beta, S0, the conv filters and the conv history.  The
 * forward is recomputed (the arguments' o, S_T and conv_state_out are written
 * again with the same values), then walked back chunk by chunk: the reverse of
 * the chunked form, with the pairs' relative decays exp(Gamma_i - Gamma_j)
 * factored per 16-token block (chunks whose decay spans are too wide for that are
 * evaluated per pair).  The optional stages are differentiated too: the
 * gradient passes back through the output stage first (o is then finished by the
 * stage in place, as kda_prefill's separate output pass does); with the
 * activations, dg and dbeta are the gradients of g and beta as given (the raw
 * gate projection, the logits).  Packed sequences too: dS_T, dS0 and
 * dconv_state are then per sequence ([n_seqs][...]); the gradients of tokens
 * outside every sequence (malformed offsets) are left undefined.  Supported: every
 * D and chunk size the forward supports.  All gradients are float32;
 * with bf16 I/O the intermediate
 * gradients pass between the kernels in bf16 (relative error of the returned
 * gradients about 4e-3 against an exact computation, at T = 4096, H = 96,
 * D = 128). */
typedef struct kda_backward_args {
  kda_prefill_args fwd; /* the forward call; its rules apply */
  const void* dO;       /* device [B][T][H][D] io dtype: gradient of o */
  const float* dS_T;    /* device [B][H][D][D] ([n_seqs][H][D][D] packed) or NULL (= zeros): gradient of S_T */
  float* dq;            /* device [B][T][H][D]: gradient of the raw q */
  float* dk;            /* device [B][T][H][D] */
  float* dv;            /* device [B][T][H][D] */
  float* dg;            /* device [B][T][H][D] */
  float* dbeta;         /* device [B][T][H] */
  float* dS0;           /* device [B][H][D][D] or NULL (not written) */
  float* dconv_w;       /* device [3][H*D][conv_k]; required iff conv_k > 0 */
  float* dconv_state;   /* device [B][3][conv_k-1][H*D] or NULL (not written) */
  /* gradients of the optional stages' parameters (ABI 4): each NULL = not written,
     and must be NULL when its stage is off */
  float* dA_log;        /* device [H]; with A_log */
  float* ddt_bias;      /* device [H*D]; with A_log */
  float* do_norm_w;     /* device [D]; with o_norm_w */
  float* do_gate;       /* device [B][T][H][D]: gradient of o_gate; with o_gate */
} kda_backward_args;

kda_status kda_validate_backward(const kda_backward_args* a);
/* Bytes of device workspace kda_prefill_backward needs (0 if invalid or T = 0). */
size_t kda_backward_workspace_bytes(const kda_backward_args* a);
/* Enqueue the recomputed forward and the backward on `stream`.  No output may
 * overlap an input or another output; the workspace overlaps nothing. */
kda_status kda_prefill_backward(const kda_backward_args* a, void* ws, size_t ws_bytes, void* stream);

/* Training: the forward kept for its backward.  kda_prefill_forward_saved gives
 * kda_prefill's results (o, S_T, conv_state_out; computed as kda_prefill_backward
 * computes them) and keeps in the workspace everything the backward would
 * otherwise recompute (the chunk records, the front end's outputs, the decay
 * sums, the state at every chunk start, and with the output stage the mixer's
 * output before it); kda_prefill_backward_saved then runs the backward alone, with
 * results identical to kda_prefill_backward's.
 *   - ws: kda_training_workspace_bytes(f) bytes, 256-byte aligned, handed from the
 *     forward to the backward untouched; the forward's inputs (q, k, v, g, beta,
 *     the filters, the previous conv state and the optional stages' parameters)
 *     must not change in between, and the backward's args.fwd must equal f.
 *   - conv_state_out may not overlap conv_state_in (KDA_ERR_ALIAS): the backward
 *     reads the previous conv state after the forward has written the new one.
 *   - T = 0: the forward hands S0 and the conv state through, the backward gives
 *     dS0 = dS_T and zero filter, history and parameter gradients; no workspace. */
size_t kda_training_workspace_bytes(const kda_prefill_args* f);
kda_status kda_prefill_forward_saved(const kda_prefill_args* f, void* ws, size_t ws_bytes,
                                     void* stream);
kda_status kda_prefill_backward_saved(const kda_backward_args* a, void* ws, size_t ws_bytes,
                                      void* stream);

/* ------------------------------------------------------------------- misc */
const char* kda_status_str(int status);
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
