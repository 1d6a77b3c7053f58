/*
 * gdn.h -- C ABI of libgdn, the MI355X (gfx950) varlen gated delta-rule hot path.
 *
 * Three operations, each one asynchronous launch sequence on the caller's HIP stream:
 *   gdn_conv1d_varlen     depthwise causal conv1d over offset-packed sequences, with a carried
 *                         (W-1)*D window per (sequence, channel)
 *   gdn_prepare_qk_gates  per-token q/k L2 normalisation plus the decay and update-rate gates
 *   gdn_scan_varlen       the gated delta-rule recurrence with a per-(sequence, head) state
 * one fusion of them for decode steps (at most one token per sequence):
 *   gdn_decode_step       gdn_conv1d_varlen then gdn_scan_varlen in a single launch
 * and variants of the same operations:
 *   gdn_conv1d_varlen_capture, gdn_scan_varlen_capture   also record the first tokens of each
 *                         sequence for speculative decoding
 *   gdn_prepare_qk_gates_strided, gdn_scan_varlen_strided   read q, k and v as separate token
 *                         streams with their own row strides
 *   gdn_scan_varlen_noalloc   gdn_scan_varlen with the library's own device scratch, for callers
 *                         that cannot allocate
 * plus gdn_scan_workspace_bytes, gdn_status_string and gdn_abi_version.
 *
 * Sources (docs.rs source pages): "onnxruntime-ep-mlx 0.31.1 src/ops/paged_ssm.rs" -- kernel strings
 * CONV, DELTA_PREPARE and DELTA, the capture strings, host functions conv(), delta() and the claim
 * predicates; "mlx-c-rust compile/gated_delta_rate_activation.rs" -- the rate-activation graph; and
 * "rlx-cpu 0.2.14 thunk/types.rs" -- Thunk::GatedDeltaNet's per-key-channel gate.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library allocates nothing,
 *     keeps no state between calls and is re-entrant (gdn_scan_varlen_noalloc alone uses a device
 *     array of the library's own, see there).  Descriptor pointers and path_used are host
 *     pointers.  Calls return as soon as the work is queued on `stream` (NULL = default stream).
 *   - Packed tokens: offsets[B+1] (int32, device) delimit sequence b as tokens
 *     [offsets[b], offsets[b+1]).  Offsets are valid iff offsets[0] == 0, offsets[B] == N and they
 *     never decrease (zero-length sequences are allowed).  Invalid offsets are detected on the
 *     device: then NO element of any output is written, and *dev_status (when dev_status is not
 *     NULL) receives GDN_ERR_OFFSETS; on valid offsets *dev_status receives GDN_OK.  The call
 *     itself still returns GDN_OK, because detection is asynchronous.
 *   - Argument errors are detected on the host before anything is launched: the call returns a
 *     negative gdn_status and writes nothing.
 *   - Pointers to tensors must be 16-byte aligned (GDN_ERR_ALIGN otherwise).
 *   - state_out may alias state_in (in-place update); no other aliasing is allowed.
 *   - Element types: GDN_F32, GDN_BF16 (bfloat16), GDN_F16 (IEEE binary16).  Outputs in a half
 *     type are rounded to nearest-even from fp32 arithmetic.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 4

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* a dimension is out of range or inconsistent */
    GDN_ERR_DTYPE = -3,       /* unknown or disallowed element type combination */
    GDN_ERR_OVERFLOW = -4,    /* a size or launch grid does not fit the index types */
    GDN_ERR_ALIGN = -5,       /* a tensor pointer is not 16-byte aligned */
    GDN_ERR_UNSUPPORTED = -6, /* valid per the op's definition but not built (see each call) */
    GDN_ERR_WORKSPACE = -7,   /* workspace missing or smaller than gdn_scan_workspace_bytes() */
    GDN_ERR_HIP = -8,         /* the HIP runtime refused a launch */
    GDN_ERR_OFFSETS = -9      /* device-detected: malformed offsets (written to *dev_status only) */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype;

/* ------------------------------------------------------------------------------------------------
 * gdn_conv1d_varlen -- paged_ssm.rs page, kernel string CONV and host fn conv().
 *
 * For sequence b with start = offsets[b], each token t of it (local index l = t - start) and each
 * channel c:
 *     y[t,c] = act( bias[c] + sum_{j<W} w[c,j] * xv(l - (W-1-j)*D) )
 * where xv(m) = x[start+m, c] for m >= 0 and state_in[b, c, L+m] for m < 0 (the carried window,
 * oldest entry first, L = (W-1)*D).  Tap W-1 multiplies the current token (causal
 * cross-correlation).  act = SiLU z/(1+e^-z) when GDN_CONV_SILU is set, else identity.  The
 * arithmetic is fp32.  The new window is the last L entries of (old window ++ the sequence's
 * tokens), copied bit-exactly (widened exactly when the window type is f32 and x is half):
 *     state_out[b, c, j] = xv(len - L + j),  j < L.
 *
 * Tensors (row-major):
 *   x          [N, C]     x_dtype                      required unless N == 0
 *   w          [C, W]     x_dtype                      required
 *   bias       [C]        x_dtype                      NULL = no bias
 *   state_in   [B, C, L]  state_dtype                  NULL = zero window
 *   y          [N, C]     x_dtype                      required unless N == 0
 *   state_out  [B, C, L]  state_dtype                  NULL = new window not produced; may alias state_in
 *   offsets    [B+1]      int32                        required
 *   dev_status [1]        int32                        NULL = no status word
 * Constraints: B >= 1, N >= 0, C >= 1, W >= 1, D >= 1, (W-1)*D and B*C within int32,
 * state_dtype is x_dtype or GDN_F32.  Widths up to 8 run on kernels that keep the taps in
 * registers; wider ones on a plain per-element form with the same arithmetic (slower).
 * ---------------------------------------------------------------------------------------------- */
#define GDN_CONV_SILU 1u

typedef struct gdn_conv_desc {
    int32_t B, N, C, W, D;
    int32_t x_dtype;     /* gdn_dtype of x, w, bias and y */
    int32_t state_dtype; /* gdn_dtype of the window: x_dtype or GDN_F32 */
    uint32_t flags;      /* GDN_CONV_SILU */
} gdn_conv_desc;

gdn_status gdn_conv1d_varlen(const gdn_conv_desc *desc, const void *x, const void *w, const void *bias,
                             const void *state_in, void *y, void *state_out, const int32_t *offsets,
                             int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * gdn_conv1d_varlen_capture -- gdn_conv1d_varlen that also records, for speculative decoding, the
 * inputs of the first tokens of each sequence (paged_ssm.rs page, CONV_CAPTURE_INIT /
 * CONV_CAPTURE_STEP, the conv node's state_update_capacity attribute and capture_count input):
 *     captured_b = max(0, min(counts[b], cap, len_b))
 *     updates[b, i, :] = x[start_b + i, :]   for i < captured_b   (bit copy)
 *     updates[b, i, :] = 0                  for captured_b <= i < cap
 * Everything else is exactly gdn_conv1d_varlen (same outputs, bit for bit).
 *   cap        slots per sequence, >= 1 (GDN_ERR_SHAPE otherwise); cap*C must fit an int32
 *   counts     [B]          int32 device, required
 *   updates    [B, cap, C]  x_dtype device, required, 16-byte aligned
 * Malformed offsets write nothing here either (the device status word reports them).
 * ---------------------------------------------------------------------------------------------- */
gdn_status gdn_conv1d_varlen_capture(const gdn_conv_desc *desc, const void *x, const void *w, const void *bias,
                                     const void *state_in, void *y, void *state_out, const int32_t *offsets,
                                     int32_t cap, const int32_t *counts, void *updates, int32_t *dev_status,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * Recurrence descriptor shared by gdn_prepare_qk_gates and gdn_scan_varlen.
 *
 * Packed token row (width C = 2*HQ*K + H*V): [q: HQ heads x K | k: HQ heads x K | v: H heads x V]
 * (paged_ssm.rs page, kernel string DELTA).  Value head h reads key head kh = h / (H/HQ)
 * (consecutive value heads share a key head).  Flags:
 *   GDN_L2NORM    q and k are scaled by 1/sqrt(sum x^2 + 1e-12) per (token, key head)
 *   GDN_SOFTPLUS  decay g = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])); without it a is a raw
 *                 log-decay and g = exp(a).  softplus(x) = max(x,0) + log1p(exp(-|x|)).
 *   GDN_SIGMOID   update rate beta = 1/(1+exp(-b)); without it beta = b.
 *   GDN_NO_RETRIEVE  the write is delta = beta*v_t, without the retrieval term k^.s: the "linear"
 *                 (no decay input) and "gated" update rules of the pages' update_rule attribute,
 *                 where the DELTA kernel string is compiled with RETRIEVE = 0.  Without this flag
 *                 the rule is "delta" (no decay input) or "gated_delta".
 *   GDN_GATE_PER_KEY  one decay per key channel: a is [N, H, K] and the decay step becomes
 *                 s[i] <- g[i]*s[i] with g[i] the gate of a[t,h,i] (A_log and dt_bias stay per
 *                 head): S <- S diag(g) before the retrieval.  The gate_per_channel form of the
 *                 GatedDeltaNet thunk (rlx-cpu thunk/types.rs page).  Fused inputs on the DECODE and
 *                 SEQ paths only: prepare, prepared scans, CHUNK, capture and gdn_decode_step reject
 *                 it (GDN_ERR_UNSUPPORTED); a must then be 16-byte aligned.
 * A NULL decay input a means g = 1; a NULL rate input b means beta = 1.  Gate arithmetic is fp32
 * (gate inputs are widened to fp32 first).  scale == 0 selects 1/sqrt(K); any other value, negative
 * included, is applied as given.
 * Constraints: B >= 1, N >= 0, HQ >= 1, H >= 1, H % HQ == 0, 1 <= K <= 256 (the pages' limit),
 * V >= 1.  Every K in that range runs on DECODE, SEQ and prepare: K = 32, 64, 128 and 256 exactly,
 * any other K on the next of those widths with the lanes' elements past K zero (element-wise row
 * accesses, so those widths are slower); CHUNK (K and V multiples of 8) and gdn_decode_step keep
 * their own width rules.
 * gate_dtype is GDN_F32 or qkv_dtype.
 * ---------------------------------------------------------------------------------------------- */
#define GDN_L2NORM 1u
#define GDN_SOFTPLUS 2u
#define GDN_SIGMOID 4u
#define GDN_NO_RETRIEVE 8u
#define GDN_GATE_PER_KEY 16u

typedef enum gdn_path {
    GDN_PATH_AUTO = 0,   /* DECODE when N <= 8*B; else CHUNK when eligible and ws_bytes suffices; else SEQ */
    GDN_PATH_DECODE = 1, /* state streamed once per call; sequences of up to 8 tokens streamed column by column */
    GDN_PATH_SEQ = 2,    /* token-sequential recurrence with the state resident in registers */
    GDN_PATH_CHUNK = 3   /* chunked WY form (chunk 64); needs a workspace and positive decays */
} gdn_path;

typedef struct gdn_scan_desc {
    int32_t B, N, HQ, H, K, V;
    int32_t qkv_dtype;  /* gdn_dtype of qkv and out */
    int32_t gate_dtype; /* gdn_dtype of a and b: GDN_F32 or qkv_dtype */
    uint32_t flags;     /* GDN_L2NORM | GDN_SOFTPLUS | GDN_SIGMOID | GDN_NO_RETRIEVE | GDN_GATE_PER_KEY */
    float scale;        /* output scale; 0 selects 1/sqrt(K), any other value is applied */
    int32_t path;       /* gdn_path */
} gdn_scan_desc;

/* ------------------------------------------------------------------------------------------------
 * Separate token streams (the *_strided entry points).  The pages' recurrence node reads one packed
 * [q | k | v] row per token and lists separate query/key/value inputs as not implemented
 * (paged_ssm.rs page, delta_claim); these entry points take the three streams apart, each with its
 * own row stride, so that q, k and v may live in separate buffers or be strided views:
 *   q row t (key head kh at kh*K):  q + t*q_stride   [HQ*K elements]
 *   k row t:                        k + t*k_stride   [HQ*K]
 *   v row t (value head h at h*V):  v + t*v_stride   [H*V]
 * Element type qkv_dtype; strides in elements, at least the row width (GDN_ERR_SHAPE); every
 * stream 16-byte aligned with rows starting 16-byte aligned (stride * element size a multiple of
 * 16; GDN_ERR_ALIGN).  Streams a call does not read may be NULL: q and k of a prepared scan, v of a
 * prepare.  A packed row of width C is q = qkv, k = qkv + HQ*K, v = qkv + 2*HQ*K, all strides C,
 * and gives bit-identical results.
 * ---------------------------------------------------------------------------------------------- */
typedef struct gdn_qkv_streams {
    const void *q;
    const void *k;
    const void *v;
    int64_t q_stride;
    int64_t k_stride;
    int64_t v_stride;
} gdn_qkv_streams;

/* ------------------------------------------------------------------------------------------------
 * gdn_prepare_qk_gates -- paged_ssm.rs page, kernel string DELTA_PREPARE; gate math also on the
 * gated_delta_rate_activation.rs page.  Token-local: no offsets.
 *   qk_out[0, t, hq, :] = q of (t, hq), normalised when GDN_L2NORM (else copied), as fp32
 *   qk_out[1, t, hq, :] = k of (t, hq), likewise
 *   gb_out[0, t, h] = g,  gb_out[1, t, h] = beta   (fp32)
 * Tensors: qkv [N, C] qkv_dtype (required); a, b [N, H] gate_dtype (NULL = absent); A_log,
 * dt_bias [H] fp32 (required when a is given and GDN_SOFTPLUS is set); qk_out [2, N, HQ, K] fp32;
 * gb_out [2, N, H] fp32.  Either output may be NULL to skip it (not both, unless N = 0).
 * ---------------------------------------------------------------------------------------------- */
gdn_status gdn_prepare_qk_gates(const gdn_scan_desc *desc, const void *qkv, const void *a, const void *b,
                                const float *A_log, const float *dt_bias, float *qk_out, float *gb_out,
                                hipStream_t stream);

/* gdn_prepare_qk_gates on separate token streams (v is not read and may be NULL). */
gdn_status gdn_prepare_qk_gates_strided(const gdn_scan_desc *desc, const gdn_qkv_streams *streams, const void *a,
                                        const void *b, const float *A_log, const float *dt_bias, float *qk_out,
                                        float *gb_out, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * gdn_scan_varlen -- paged_ssm.rs page, kernel string DELTA (and the chunked variant the host fn
 * delta() selects).  For each sequence b, value head h, value column v, with s = state_in[b,h,v,:]
 * (a K-vector; zeros when state_in is NULL), over the sequence's tokens t in order:
 *     s <- g*s;  r = k^.s;  delta = beta*(v_t - r);  s <- s + delta*k^;  out[t,h,v] = scale*(q^.s)
 * (r = 0 with GDN_NO_RETRIEVE)
 * then state_out[b,h,v,:] = s.  q^, k^, g, beta are either computed in-kernel from qkv, a, b,
 * A_log, dt_bias and the flags ("fused"), or read from a prior gdn_prepare_qk_gates call when both
 * qk_prep and gb_prep are given ("prepared"; then a, b, A_log, dt_bias and the flags are unused).
 * v_t always comes from qkv.  All recurrence arithmetic is fp32.
 *
 * Tensors:
 *   qkv        [N, C]        qkv_dtype   required
 *   qk_prep    [2, N, HQ, K] fp32        NULL = fused (must be NULL together with gb_prep)
 *   gb_prep    [2, N, H]     fp32
 *   a          [N, H]        gate_dtype  NULL = absent (fused mode); [N, H, K] with GDN_GATE_PER_KEY
 *   b          [N, H]        gate_dtype  NULL = absent (fused mode)
 *   A_log, dt_bias [H]       fp32        required in fused mode when a is given with GDN_SOFTPLUS
 *   state_in   [B, H, V, K]  fp32        NULL = zero state
 *   out        [N, H, V]     qkv_dtype   required unless N == 0
 *   state_out  [B, H, V, K]  fp32        NULL = final state not produced; may alias state_in
 *   offsets    [B+1]         int32       required
 *   workspace  device scratch of ws_bytes bytes, needed only by GDN_PATH_CHUNK (query the size
 *              with gdn_scan_workspace_bytes); may be NULL otherwise
 *   dev_status [1] int32 (NULL ok); path_used: HOST int32 receiving the gdn_path that ran (NULL ok)
 * GDN_PATH_CHUNK requires fused mode with a decay input (not needed when N = 0) and GDN_SOFTPLUS
 * (so every decay is finite and positive), GDN_L2NORM, the retrieval term (no GDN_NO_RETRIEVE),
 * bf16 or fp16 qkv, and K and V multiples of 8 (the chunked rule of the paged_ssm.rs page's host
 * fn delta(): K != V included); otherwise GDN_ERR_UNSUPPORTED.  K runs on the next of 64, 128 and
 * 256 and V in parts of at most 128 columns (one block each), with the keys and columns past K and
 * V zero.  Long sequences are cut into segments that run in parallel at K <= 64 with V <= 64 and at
 * 65 <= K <= 128 with 33 <= V <= 128; other widths run each sequence in one piece.  Its
 * intra-chunk contractions run on bf16 matrix cores with fp32 accumulation (the state itself
 * stays fp32).
 * ---------------------------------------------------------------------------------------------- */
gdn_status gdn_scan_varlen(const gdn_scan_desc *desc, const void *qkv, const float *qk_prep, const float *gb_prep,
                           const void *a, const void *b, const float *A_log, const float *dt_bias,
                           const float *state_in, void *out, float *state_out, const int32_t *offsets,
                           void *workspace, size_t ws_bytes, int32_t *dev_status, int32_t *path_used,
                           hipStream_t stream);

/* gdn_scan_varlen on separate token streams: every path, flag and argument as above, with qkv
 * replaced by the three streams (q and k unread, and may be NULL, with prepared inputs). */
gdn_status gdn_scan_varlen_strided(const gdn_scan_desc *desc, const gdn_qkv_streams *streams, const float *qk_prep,
                                   const float *gb_prep, const void *a, const void *b, const float *A_log,
                                   const float *dt_bias, const float *state_in, void *out, float *state_out,
                                   const int32_t *offsets, void *workspace, size_t ws_bytes, int32_t *dev_status,
                                   int32_t *path_used, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * gdn_scan_varlen_capture -- gdn_scan_varlen that also records, for speculative decoding, the
 * rank-one updates of the first tokens of each sequence (paged_ssm.rs page, DELTA_CAPTURE_INIT /
 * DELTA_CAPTURE_STEP, the recurrence node's state_update_capacity attribute, capture_count and
 * state_update_active inputs and compact capsule output).  With
 *     captured_b = (active != NULL && active[0] == 0) ? 0 : max(0, min(counts[b], cap, len_b))
 * the fp32 capsule row of sequence b is [cap*H g | cap*HQ*K k^ | cap*H*V delta]:
 *     capsule[b, i*H + h]                          = g of token start_b + i, head h
 *     capsule[b, cap*H + (i*HQ + kh)*K + j]        = k^[j] of that token, key head kh
 *     capsule[b, cap*(H + HQ*K) + (i*H + h)*V + v] = delta = beta*(v_t - r) of column (h, v)
 * for i < captured_b, and 0 in every slot i >= captured_b.  Replaying
 *     S_i = g_i * S_{i-1} + delta_i k^_i^T   (S_0 = state_in, rows v, columns over K)
 * for i < captured_b gives the state after those tokens, which is how a speculative decoder rolls
 * the state forward to the accepted prefix.  Outputs and final state are those of gdn_scan_varlen.
 *   cap        slots per sequence, >= 1 (GDN_ERR_SHAPE); cap*(H + HQ*K + H*V) must fit an int32
 *              (GDN_ERR_OVERFLOW)
 *   counts     [B] int32 device, required
 *   active     [1] int32 device, NULL = always active
 *   capsule    [B, cap*(H + HQ*K + H*V)] fp32 device, required, 16-byte aligned
 * Recorded by every path.  CHUNK records from a sequence's first chunk of 64 tokens, so it takes
 * cap <= 64 (a larger cap sends AUTO to SEQ, and an explicit GDN_PATH_CHUNK is
 * GDN_ERR_UNSUPPORTED); its delta slots carry the chunked form's rounding (bf16 operands).
 * Malformed offsets write nothing.
 * ---------------------------------------------------------------------------------------------- */
gdn_status gdn_scan_varlen_capture(const gdn_scan_desc *desc, const void *qkv, const float *qk_prep,
                                   const float *gb_prep, const void *a, const void *b, const float *A_log,
                                   const float *dt_bias, const float *state_in, void *out, float *state_out,
                                   const int32_t *offsets, int32_t cap, const int32_t *counts, const int32_t *active,
                                   float *capsule, void *workspace, size_t ws_bytes, int32_t *dev_status,
                                   int32_t *path_used, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * gdn_decode_step -- a decode step in one launch: exactly gdn_conv1d_varlen(conv, x -> y) followed
 * by gdn_scan_varlen(scan, y, fused mode, DECODE path), with bit-identical outputs, new window and
 * final state, for calls where every sequence holds at most one token.  y is not materialised.
 * (paged_ssm.rs page, kernel strings CONV and DELTA; the gated_delta_rate_activation.rs page names
 * launches per decode step as this layer's cost.)
 *
 * Tensors are those of the two calls it replaces, with the same layouts, dtypes and NULL rules:
 *   x [N, C], conv_w [C, W], conv_bias [C] (NULL = none), conv_state_in / conv_state_out
 *   [B, C, L] (window; NULL in = zeros, NULL out = not produced, may alias), a, b [N, H],
 *   A_log, dt_bias [H], state_in / state_out [B, H, V, K] fp32 (may alias), out [N, H, V].
 * The descriptors must agree: conv->B == scan->B, conv->N == scan->N,
 * conv->C == 2*HQ*K + H*V, conv->x_dtype == scan->qkv_dtype (GDN_ERR_SHAPE / GDN_ERR_DTYPE);
 * scan->path is GDN_PATH_AUTO or GDN_PATH_DECODE.  Built for K in {32, 64, 128, 256},
 * V % 4 == 0, (W-1)*D <= 4 and (2K + (H/HQ)*V) * 4 <= 65536 bytes; N > B is rejected
 * (GDN_ERR_UNSUPPORTED).  On the device, malformed offsets give *dev_status = GDN_ERR_OFFSETS
 * and a sequence with more than one token gives GDN_ERR_UNSUPPORTED; in both cases nothing is
 * written.
 * ---------------------------------------------------------------------------------------------- */
gdn_status gdn_decode_step(const gdn_conv_desc *conv, const gdn_scan_desc *scan, const void *x, const void *conv_w,
                           const void *conv_bias, const void *conv_state_in, void *conv_state_out, const void *a,
                           const void *b, const float *A_log, const float *dt_bias, const float *state_in, void *out,
                           float *state_out, const int32_t *offsets, int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------------------------------
 * gdn_scan_varlen_noalloc -- gdn_scan_varlen for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * paths, results (bit for bit) and errors as gdn_scan_varlen on a packed row, without the workspace
 * arguments: the chunked path's workspace is the library's own device array of
 * GDN_NOALLOC_SCRATCH_BYTES, placed once per device by the HIP runtime and kept until the process
 * ends.  The call allocates nothing.
 *   - AUTO takes the chunked path only when its workspace fits the array; an explicit
 *     GDN_PATH_CHUNK whose workspace (gdn_scan_workspace_bytes) exceeds it returns
 *     GDN_ERR_WORKSPACE.
 *   - The array of the CURRENT device is used (hipGetDevice), so `stream` must belong to it.  Its
 *     address is looked up on the first call on each device (GDN_ERR_HIP if that fails).
 *   - Every call on one device shares that device's array: calls that overlap in time on one device
 *     (other streams, other host threads) race and must be serialised by the caller.  The array
 *     keeps the last call's contents; nothing in it needs to start at zero.
 * ---------------------------------------------------------------------------------------------- */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gdn_status gdn_scan_varlen_noalloc(const gdn_scan_desc *desc, const void *qkv, const float *qk_prep,
                                   const float *gb_prep, const void *a, const void *b, const float *A_log,
                                   const float *dt_bias, const float *state_in, void *out, float *state_out,
                                   const int32_t *offsets, int32_t *dev_status, int32_t *path_used, hipStream_t stream);

/* Workspace bytes gdn_scan_varlen needs for `desc` (with its path resolved as AUTO would);
 * 0 when the resolved path needs none.  Returns the same argument errors as gdn_scan_varlen. */
gdn_status gdn_scan_workspace_bytes(const gdn_scan_desc *desc, size_t *bytes);

/* Static description of a status code; never NULL. */
const char *gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
