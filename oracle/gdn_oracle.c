/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the varlen gated delta-rule hot path,
 * computed in fp64.  Only the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header, table or helper with the HIP library: the
 * element decoders, the offsets check, the gate formulas and the recurrence below are written
 * out independently from the definitions on the source pages.
 *
 * Sources (docs.rs source pages; cited by page and named item):
 *   [conv]    onnxruntime-ep-mlx 0.31.1, src/ops/paged_ssm.rs -- kernel string CONV and host fn conv()
 *   [prep]    same page -- kernel string DELTA_PREPARE
 *   [delta]   same page -- kernel string DELTA and host fn delta()
 *   [rates]   mlx-c-rust, compile/gated_delta_rate_activation.rs -- the rate-activation graph builder
 *   [thunk]   rlx-cpu 0.2.14, thunk/types.rs -- Thunk::GatedDeltaNet (its gate_per_channel field)
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - offsets are valid iff offsets[0]==0, offsets[B]==N and offsets never decrease; an invalid
 *     call writes nothing at all (the pages' kernels check the endpoints and each sequence's own
 *     pair per thread; the strict whole-call reading is the plainest one that is deterministic).
 *   - a NULL initial state means zeros.
 *   - the epsilon of the q/k L2 norm is added to the sum of squares inside the square root.
 *   - softplus(x) = max(x,0) + log1p(exp(-|x|)), i.e. logaddexp(x, 0).
 *   - every value is decoded exactly to double first; nothing is rounded on the way out.
 *
 * Dtype codes used by this file: 0 = float32, 1 = bfloat16, 2 = float16 (IEEE binary16).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_F16 2

/* ---- element decoders: bit layouts of IEEE binary32, bfloat16 and IEEE binary16 ---------------- */

static double dec_bf16_bits(uint16_t h) {
    /* bfloat16 is the upper half of an IEEE binary32 word. */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double dec_f16_bits(uint16_t h) {
    /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = m ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static double dec(const void *p, int dtype, size_t i) {
    switch (dtype) {
    case OR_F32: return (double)((const float *)p)[i];
    case OR_BF16: return dec_bf16_bits(((const uint16_t *)p)[i]);
    case OR_F16: return dec_f16_bits(((const uint16_t *)p)[i]);
    default: return NAN;
    }
}

/* Exposed so the tests can pin the decoders against library conversions. */
double gdn_oracle_decode(const void *p, int dtype, long long i) { return dec(p, dtype, (size_t)i); }

/* ---- offsets ------------------------------------------------------------------------------------ */

/* 1 if offsets[0..B] describe B packed sequences covering tokens [0, N), else 0.
 * [conv]/[delta]: a sequence is processed only when offsets[0]==0, offsets[B]==N and
 * 0 <= start <= end <= N; read strictly over the whole call. */
int gdn_oracle_offsets_valid(const int32_t *offsets, int B, int N) {
    if (B < 1 || offsets == NULL) return 0;
    if (offsets[0] != 0 || offsets[B] != N) return 0;
    for (int i = 0; i < B; ++i) {
        if (offsets[i] < 0 || offsets[i] > N) return 0;
        if (offsets[i + 1] < offsets[i]) return 0;
    }
    return 1;
}

/* ---- varlen depthwise causal conv1d with a carried window -------------------------------------- */

/* [conv]: for sequence b, channel c and each token t of the sequence (local index l = t - start),
 *   y[t,c] = act( bias[c] + sum_{j<W} w[c,j] * xv(l - (W-1-j)*D) ),
 * where xv(m) is the input token start+m when m >= 0 and the carried window entry
 * state_in[b,c,L+m] otherwise (L = (W-1)*D, oldest entry first).  act is SiLU z/(1+e^-z) when
 * silu != 0, else the identity.  The new window is the last L entries of (old window ++ the
 * sequence's tokens): state_out[b,c,j] = xv(len - L + j).
 *
 * Shapes: x, y [N,C]; w [C,W]; bias [C] or NULL; state_in, state_out [B,C,L] (state_in NULL ->
 * zeros; state_out NULL -> not produced).  x, w and bias use x_dtype, the window uses state_dtype.
 * Returns 0 on success, 1 when the offsets are malformed (then nothing is written). */
int gdn_oracle_conv(int B, int N, int C, int W, int D, int x_dtype, int state_dtype, int silu,
                    const void *x, const void *w, const void *bias, const void *state_in,
                    const int32_t *offsets, double *y, double *state_out) {
    if (!gdn_oracle_offsets_valid(offsets, B, N)) return 1;
    const long long L = (long long)(W - 1) * D;
    for (int b = 0; b < B; ++b) {
        const int start = offsets[b];
        const int len = offsets[b + 1] - start;
        for (int c = 0; c < C; ++c) {
            const size_t wbase = (size_t)b * C + c; /* window row of (b, c) */
            for (int l = 0; l < len; ++l) {
                double acc = bias ? dec(bias, x_dtype, (size_t)c) : 0.0;
                for (int j = 0; j < W; ++j) {
                    long long m = (long long)l - (long long)(W - 1 - j) * D;
                    double xv;
                    if (m >= 0)
                        xv = dec(x, x_dtype, (size_t)(start + m) * C + c);
                    else
                        xv = state_in ? dec(state_in, state_dtype, (size_t)(wbase * L + L + m)) : 0.0;
                    acc += dec(w, x_dtype, (size_t)c * W + j) * xv;
                }
                if (silu) acc = acc / (1.0 + exp(-acc));
                y[(size_t)(start + l) * C + c] = acc;
            }
            if (state_out) {
                for (long long j = 0; j < L; ++j) {
                    long long m = (long long)len - L + j;
                    double v;
                    if (m >= 0)
                        v = dec(x, x_dtype, (size_t)(start + m) * C + c);
                    else
                        v = state_in ? dec(state_in, state_dtype, (size_t)(wbase * L + L + m)) : 0.0;
                    state_out[wbase * L + j] = v;
                }
            }
        }
    }
    return 0;
}

/* ---- q/k normalisation and the gate / rate activations ----------------------------------------- */

/* [prep], [delta] and [rates]: decay g from the decay input x of head h:
 *   softplus on: g = exp( -exp(A_log[h]) * softplus(x + dt_bias[h]) )
 *   softplus off: x is a raw log-decay and g = exp(x). */
static double decay_gate(double x, int softplus, double a_log, double dtb) {
    if (softplus) {
        double z = x + dtb;
        double sp = (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
        x = -exp(a_log) * sp;
    }
    return exp(x);
}

/* [prep], [delta] and [rates]: update rate beta = sigmoid(x) = 1/(1+e^-x), or x itself when raw. */
static double rate_gate(double x, int sigmoid) { return sigmoid ? 1.0 / (1.0 + exp(-x)) : x; }

/* [prep]: for every token t and key head hq, the q and k vectors (packed row [q | k | v], q of head
 * hq at hq*K, k at HQ*K + hq*K) are scaled by 1/sqrt(sum x^2 + 1e-12) when l2norm != 0 and passed
 * unchanged otherwise; qk_out is [2,N,HQ,K] (q plane then k plane).  For every token t and value
 * head h, gb_out[0,t,h] = g (1 when a is NULL) and gb_out[1,t,h] = beta (1 when b is NULL); gb_out
 * is [2,N,H].  a and b are [N,H] in gate_dtype; A_log and dt_bias are [H] float32 (used only with
 * softplus).  Either output pointer may be NULL. */
void gdn_oracle_prepare(int N, int HQ, int H, int K, int V, int qkv_dtype, int gate_dtype, int l2norm,
                        int softplus, int sigmoid, const void *qkv, const void *a, const void *b,
                        const float *A_log, const float *dt_bias, double *qk_out, double *gb_out) {
    const size_t C = (size_t)2 * HQ * K + (size_t)H * V;
    if (qk_out) {
        for (int t = 0; t < N; ++t) {
            for (int plane = 0; plane < 2; ++plane) {
                for (int hq = 0; hq < HQ; ++hq) {
                    const size_t src = (size_t)t * C + (size_t)plane * HQ * K + (size_t)hq * K;
                    double ss = 0.0;
                    for (int i = 0; i < K; ++i) {
                        double v = dec(qkv, qkv_dtype, src + i);
                        ss += v * v;
                    }
                    const double r = l2norm ? 1.0 / sqrt(ss + 1e-12) : 1.0;
                    double *dst = qk_out + (((size_t)plane * N + t) * HQ + hq) * K;
                    for (int i = 0; i < K; ++i) dst[i] = dec(qkv, qkv_dtype, src + i) * r;
                }
            }
        }
    }
    if (gb_out) {
        for (int t = 0; t < N; ++t) {
            for (int h = 0; h < H; ++h) {
                const size_t i = (size_t)t * H + h;
                double g = 1.0, beta = 1.0;
                if (a)
                    g = decay_gate(dec(a, gate_dtype, i), softplus, softplus ? (double)A_log[h] : 0.0,
                                   softplus ? (double)dt_bias[h] : 0.0);
                if (b) beta = rate_gate(dec(b, gate_dtype, i), sigmoid);
                gb_out[i] = g;
                gb_out[(size_t)N * H + i] = beta;
            }
        }
    }
}

/* [conv capture]: the raw inputs of the first tokens of each sequence, for speculative decoding
 * (paged_ssm.rs page, CONV_CAPTURE_INIT / CONV_CAPTURE_STEP): with captured = max(0, min(counts[b],
 * cap, len_b)), updates[b,i,c] = x[start_b + i, c] for i < captured and 0 for captured <= i < cap.
 * updates is [B, cap, C] decoded to fp64.  Returns 0, or 1 when the offsets are malformed. */
int gdn_oracle_conv_capture(int B, int N, int C, int cap, int x_dtype, const void *x, const int32_t *offsets,
                            const int32_t *counts, double *updates) {
    if (!gdn_oracle_offsets_valid(offsets, B, N)) return 1;
    for (int b = 0; b < B; ++b) {
        const int start = offsets[b], len = offsets[b + 1] - start;
        int captured = counts[b] < cap ? counts[b] : cap;
        if (captured > len) captured = len;
        if (captured < 0) captured = 0;
        for (int i = 0; i < cap; ++i)
            for (int c = 0; c < C; ++c)
                updates[((size_t)b * cap + i) * C + c] = i < captured ? dec(x, x_dtype, (size_t)(start + i) * C + c) : 0.0;
    }
    return 0;
}

/* ---- the gated delta-rule recurrence ------------------------------------------------------------ */

/* [delta]: for each sequence b, value head h (key head kh = h / (H/HQ)) and value column v, the
 * state s = state_in[b,h,v,:] (a K-vector; zeros when state_in is NULL) is carried through the
 * sequence's tokens in order:
 *     s <- g * s
 *     r  = k^ . s
 *     delta = beta * (v_t - r)
 *     s <- s + delta * k^
 *     out[t,h,v] = scale * (q^ . s)
 * with q^, k^, g, beta as produced by gdn_oracle_prepare.  The final s is state_out[b,h,v,:].
 * Capture (paged_ssm.rs page, DELTA_CAPTURE_INIT / DELTA_CAPTURE_STEP), when capsule is not NULL:
 * per sequence b the first captured = (active && !active[0]) ? 0 : max(0, min(counts[b], cap, len_b))
 * steps are recorded in capsule[b] = [cap*H g | cap*HQ*K k^ | cap*H*V delta] (slot i: g of (i, h) at
 * i*H + h; k^ of (i, kh) at cap*H + (i*HQ + kh)*K; delta of (i, h, v) at cap*(H + HQ*K) +
 * (i*H + h)*V + v); slots from captured on are 0.  delta is the written value beta*(v_t - r), so
 * S_i = g_i S_{i-1} + delta_i k^_i^T replays the recurrence.
 * retrieve == 0 drops the retrieval term (delta = beta * v_t): the "linear" and "gated" update rules
 * of the pages' update_rule attribute, which the DELTA kernel string compiles with RETRIEVE = 0
 * (the rule's decay side is the presence of the decay input, as for the other rules).
 * gate_per_key != 0 gives every key channel its own decay (the rlx-cpu thunk/types.rs page,
 * Thunk::GatedDeltaNet with gate_per_channel: g shaped like the keys): a is [N,H,K] and the first step
 * becomes s[i] <- g_i * s[i] with g_i = decay_gate(a[t,h,i]) (A_log and dt_bias stay per head);
 * in matrix form S <- S diag(g) (I - beta k^ k^T) + beta v k^T.  Not combined with a capture.
 * scale == 0 selects 1/sqrt(K); any other value, negative included, is applied as given (host fn
 * delta(): a zero scale attribute means 1/sqrt(K)).
 * Layouts: qkv [N, 2*HQ*K + H*V]; out [N,H,V]; state [B,H,V,K] float32 in, fp64 out.
 * Returns 0 on success, 1 when the offsets are malformed (then nothing is written), 2 when out of
 * memory, 3 for a per-key gate with a capture.  Parallel over independent (b, h) pairs with OpenMP
 * when built with it. */
int gdn_oracle_scan(int B, int N, int HQ, int H, int K, int V, int qkv_dtype, int gate_dtype,
                    int l2norm, int softplus, int sigmoid, int retrieve, int gate_per_key, double scale,
                    const void *qkv,
                    const void *a, const void *b, const float *A_log, const float *dt_bias,
                    const float *state_in, const int32_t *offsets, double *out, double *state_out,
                    const int32_t *counts, const int32_t *active, int cap, double *capsule) {
    if (!gdn_oracle_offsets_valid(offsets, B, N)) return 1;
    if (gate_per_key && a && capsule) return 3;
    if (scale == 0.0) scale = 1.0 / sqrt((double)K);
    const size_t C = (size_t)2 * HQ * K + (size_t)H * V;
    const void *a_head = gate_per_key ? NULL : a; /* per-head decay input, evaluated by prepare */
    const int G = H / HQ;
    double *qk = (double *)malloc(sizeof(double) * ((size_t)2 * N * HQ * K + 1));
    double *gb = (double *)malloc(sizeof(double) * ((size_t)2 * N * H + 1));
    if (!qk || !gb) {
        free(qk);
        free(gb);
        return 2;
    }
    gdn_oracle_prepare(N, HQ, H, K, V, qkv_dtype, gate_dtype, l2norm, softplus, sigmoid, qkv, a_head, b,
                       A_log, dt_bias, qk, gb);
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long long bh = 0; bh < (long long)B * H; ++bh) {
        const int bb = (int)(bh / H), h = (int)(bh % H);
        const int kh = h / G;
        const int start = offsets[bb], end = offsets[bb + 1];
        int captured = 0;
        double *cb = NULL;
        if (capsule) {
            captured = counts[bb] < cap ? counts[bb] : cap;
            if (captured > end - start) captured = end - start;
            if (captured < 0 || (active && active[0] == 0)) captured = 0;
            cb = capsule + (size_t)bb * cap * ((size_t)H + (size_t)HQ * K + (size_t)H * V);
            for (int i = 0; i < cap; ++i) {  /* every slot of (b, h), then filled below */
                cb[(size_t)i * H + h] = 0.0;
                if (h == kh * G)
                    for (int j = 0; j < K; ++j) cb[(size_t)cap * H + ((size_t)i * HQ + kh) * K + j] = 0.0;
                for (int v = 0; v < V; ++v) cb[(size_t)cap * (H + (size_t)HQ * K) + ((size_t)i * H + h) * V + v] = 0.0;
            }
        }
        double *s = (double *)malloc(sizeof(double) * (size_t)K);
        if (!s) {
            failed = 1;
            continue;
        }
        for (int v = 0; v < V; ++v) {
            const size_t col = ((size_t)bb * H + h) * V + v;
            for (int i = 0; i < K; ++i) s[i] = state_in ? (double)state_in[col * K + i] : 0.0;
            for (int t = start; t < end; ++t) {
                const double *qh = qk + ((size_t)t * HQ + kh) * K;
                const double *kk = qk + (((size_t)N + t) * HQ + kh) * K;
                const double g = gb[(size_t)t * H + h];
                const double beta = gb[((size_t)N + t) * H + h];
                const double vt = dec(qkv, qkv_dtype, (size_t)t * C + (size_t)2 * HQ * K + (size_t)h * V + v);
                if (gate_per_key && a) {
                    for (int i = 0; i < K; ++i)
                        s[i] *= decay_gate(dec(a, gate_dtype, ((size_t)t * H + h) * K + i), softplus,
                                           softplus ? (double)A_log[h] : 0.0, softplus ? (double)dt_bias[h] : 0.0);
                } else {
                    for (int i = 0; i < K; ++i) s[i] *= g;
                }
                double r = 0.0;
                if (retrieve)
                    for (int i = 0; i < K; ++i) r += kk[i] * s[i];
                const double delta = beta * (vt - r);
                const int slot = t - start;
                if (cb && slot < captured) {
                    if (v == 0) cb[(size_t)slot * H + h] = g;
                    if (v == 0 && h == kh * G)
                        for (int j = 0; j < K; ++j) cb[(size_t)cap * H + ((size_t)slot * HQ + kh) * K + j] = kk[j];
                    cb[(size_t)cap * (H + (size_t)HQ * K) + ((size_t)slot * H + h) * V + v] = delta;
                }
                for (int i = 0; i < K; ++i) s[i] += delta * kk[i];
                double o = 0.0;
                for (int i = 0; i < K; ++i) o += qh[i] * s[i];
                out[((size_t)t * H + h) * V + v] = scale * o;
            }
            if (state_out)
                for (int i = 0; i < K; ++i) state_out[col * K + i] = s[i];
        }
        free(s);
    }
    free(qk);
    free(gb);
    return failed ? 2 : 0;
}

/* Threads for the following calls (test infrastructure: timing the oracle at a chosen width). */
void gdn_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of OpenMP threads the scan will use (1 without OpenMP). */
int gdn_oracle_threads(void) {
#ifdef _OPENMP
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}
