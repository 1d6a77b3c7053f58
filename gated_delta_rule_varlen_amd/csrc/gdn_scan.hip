// gdn_scan.hip -- gated delta-rule recurrence, DECODE path: token-sequential form with the state
// streamed once per call (gfx950, wave64).  Correct for any sequence lengths; tiled for many short
// sequences (the prefill path with LDS-staged token chunks is gdn_seq.hip).
//
// Operation: paged_ssm.rs page, kernel string DELTA (see gdn.h).  Every value column (b, h, v) is an
// independent recurrence over a K-vector s.  Work mapping:
//
//   * a column is owned by a group of LPC adjacent lanes; lane j of the group holds the K-indices
//     4*(j + LPC*i) + e (i < K/(4*LPC), e < 4), so every 16-byte state access of a group is one
//     contiguous 16*LPC-byte segment and the state of a block streams with perfectly coalesced
//     loads and stores;
//   * a lane group carries CPL columns of the same head, a wave 64/LPC groups, a block NW waves
//     (one column tile per wave);
//     blocks are laid out (sequence, head, column tile) and re-mapped so that the blocks of one
//     head land on one XCD (they read the same q/k rows through that XCD's L2);
//   * per token the two state dot products k.s and q.s of the OLD state are computed together, then
//     reduced over the group with a 4-step DPP butterfly (the page's 32-wide simd_sum becomes a
//     16-lane row reduction).  Using
//         r = g (k^.s),  delta = beta (v - r),  q^.s' = g (q^.s) + delta (q^.k^)
//     the readout needs no second reduction after the update, which halves the serial chain;
//   * "fused" instances normalise q/k and evaluate the gates in-kernel from the raw inputs (one
//     launch per decode step: no prepare pass, no fp32 q/k round trip through HBM); "prepared"
//     instances read the fp32 outputs of gdn_prepare_qk_gates;
//   * the next token's operands are loaded while the current token is computed;
//   * a block whose sequence has exactly one token (the decode step) streams its columns instead:
//     token operands first, then the state columns of a group with all their loads in flight, each
//     column reduced, updated, written back and its output taken in turn, so reads and writes of
//     the state interleave.  Same arithmetic in the same order, so the results are bit-identical;
//   * "SHORT" instances serve calls with more tokens than sequences.  A block whose sequence has
//     2 .. GDN_DECODE_SHORT tokens (a speculative verification step, a short prefill) first stages
//     the tokens' normalised q and k, gates, q^.k^ and its columns' v in LDS, once per block instead
//     of once per lane group, then carries its whole column tile through the tokens with the state
//     kept as s = c * s' (c the product of the decays so far, uniform over the block), so that a
//     token costs the two dot products and one fused multiply-add per state element (per-key
//     decays are staged per channel too and applied to the tile directly);
//   * with a per-key-channel decay (GDN_GATE_PER_KEY; "PK" instances) thread i of the block
//     evaluates the decay of key channel i once per token into LDS (every wave of a block serves
//     the same head), and each lane decays its state slice before the two dot products
//     (s' = g o s), so r and the readout use the decayed state directly;
//   * with capture (speculative decoding: paged_ssm.rs page, DELTA_CAPTURE_INIT / _STEP) the first
//     captured tokens of a sequence also record g (one lane of the head's first block), k^ (the
//     first lane group of that block, for the first value head of each key head) and delta (the
//     lane that writes the column's output); the slots after them are zeroed by the same lanes.
//
// DECODE instances stream the state with non-temporal loads/stores (read once, written once).
// Key widths other than 32, 64, 128 and 256 run on the next compiled width ("KX = false"
// instances): the lanes' elements past K read as zero and are never written, so dot products,
// norms and updates are those of the K-wide rows.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

// Single-token decode blocks stream their state columns with this many columns of loads in flight
// (0 keeps the whole tile in registers as for longer sequences).  Measured at B=256, H=32,
// K=V=128: streaming all 4 columns of a group with each column stored as soon as it is updated
// moves the state at 6.2 TB/s, against 5.7 TB/s for load-all / compute / store-all at 8 columns.
#ifndef GDN_DECODE_STREAM
#define GDN_DECODE_STREAM 4
#endif
// Longest sequence the SHORT instances carry through their staged-operand form.
#ifndef GDN_DECODE_SHORT
#define GDN_DECODE_SHORT kDecodeShortTokens
#endif

namespace gdn {
namespace {

struct ScanArgs {
    TokenStreams x;
    const float* qk_prep;
    const float* gb_prep;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    const float* state_in;  // not restrict: may alias state_out
    void* out;
    float* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    int B, N, HQ, H, K, V, G;
    int gate_dtype;
    uint32_t flags;
    float scale;
    int n_vtiles;   // column tiles per (sequence, head)
    int n_blocks;   // grid size
    int cap;                // capture slots per sequence (0 = no capture)
    const int32_t* counts;  // [B]
    const int32_t* active;  // [1] or NULL
    float* capsule;         // [B, cap*(H + HQ*K + H*V)]
};

// Operands of one token as seen by one lane.
template <int EPL, int CPL, bool PK>
struct TokenOps {
    float q[EPL];
    float k[EPL];
    float v[CPL];
    float ga;               // prepared: g; fused: raw decay input (0 when absent; unused with PK)
    float gb;               // prepared: beta; fused: raw rate input (0 when absent)
    float gkr;              // PK: raw decay input of key channel threadIdx.x (threads below K)
};

template <typename T, int K, int LPC, int CPL, bool PREP, bool PK, bool KX>
__device__ __forceinline__ void load_token(const ScanArgs& p, int t, int h, int kh, int gl, int vbase,
                                           TokenOps<K / LPC, CPL, PK>& o) {
    constexpr int EPL = K / LPC;
    using TS = typename T::storage;
    const int Kr = KX ? K : p.K;
    if constexpr (PREP) {
        const float* qp = p.qk_prep + ((size_t)t * p.HQ + kh) * Kr;
        const float* kp = p.qk_prep + (((size_t)p.N + t) * p.HQ + kh) * Kr;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
            const f32x4 qv = ld_row4<KX, false>(qp, 4 * (gl + LPC * i), Kr);
            const f32x4 kv = ld_row4<KX, false>(kp, 4 * (gl + LPC * i), Kr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o.q[4 * i + e] = qv[e];
                o.k[4 * i + e] = kv[e];
            }
        }
        o.ga = p.gb_prep[(size_t)t * p.H + h];
        o.gb = p.gb_prep[((size_t)p.N + t) * p.H + h];
    } else {
        const TS* qp = static_cast<const TS*>(p.x.q) + (size_t)t * p.x.sq + (size_t)kh * Kr;
        const TS* kp = static_cast<const TS*>(p.x.k) + (size_t)t * p.x.sk + (size_t)kh * Kr;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
            const f32x4 qv = ld_in4<T, KX>(qp, 4 * (gl + LPC * i), Kr);
            const f32x4 kv = ld_in4<T, KX>(kp, 4 * (gl + LPC * i), Kr);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o.q[4 * i + e] = qv[e];
                o.k[4 * i + e] = kv[e];
            }
        }
        const size_t gi = (size_t)t * p.H + h;
        if constexpr (PK) {
            o.ga = 0.0f;
            o.gkr = (int)threadIdx.x < Kr ? load_any(p.a, p.gate_dtype, gi * Kr + threadIdx.x) : 0.0f;
        } else {
            o.ga = p.a ? load_any(p.a, p.gate_dtype, gi) : 0.0f;
        }
        o.gb = p.b ? load_any(p.b, p.gate_dtype, gi) : 0.0f;
    }
    const TS* vp = static_cast<const TS*>(p.x.v) + (size_t)t * p.x.sv + (size_t)h * p.V + vbase;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o.v[c] = (vbase + c < p.V) ? to_f32<T>(vp[c]) : 0.0f;
}

template <typename T, int K, int LPC, int CPL, int NW, bool PREP, bool NT, bool PK, bool SHORT, bool KX>
__global__ __launch_bounds__(64 * NW) void scan_kernel(ScanArgs p) {
    static_assert(!(PK && PREP), "the per-key decay is evaluated in-kernel from raw inputs");
    // K is the compiled key width; rows are Kr wide (Kr < K: the lanes' elements past Kr are zero)
    const int Kr = KX ? K : p.K;
    constexpr int EPL = K / LPC;  // state elements per lane per column
    static_assert(EPL % 4 == 0, "whole 16-byte chunks per lane");
    constexpr int GPW = 64 / LPC;  // lane groups per wave
    constexpr int WC = GPW * CPL;  // columns per wave; a block covers NW * WC
    using TS = typename T::storage;

    static_assert(!PK || 64 * NW >= K, "one thread per key channel stages the decays");
    __shared__ __align__(16) float gks[PK ? K : 1];  // PK: the token's decay per key channel

    const bool malformed = offsets_malformed(p.offsets, p.B, p.N);
    report_status(p.dev_status, malformed);
    if (malformed) return;

    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, p.G * p.n_vtiles);
    const int vt = blk % p.n_vtiles;
    const int bh = blk / p.n_vtiles;
    const int h = bh % p.H;
    const int b = bh / p.H;
    const int kh = h / p.G;
    const int wave = (int)threadIdx.x / 64;
    const int lane = (int)threadIdx.x % 64;
    const int grp = lane / LPC, gl = lane % LPC;
    const int vbase = (vt * NW + wave) * WC + grp * CPL;
    const size_t col0 = ((size_t)b * p.H + h) * p.V;

    const int start = p.offsets[b], end = p.offsets[b + 1];
    const bool l2 = (p.flags & GDN_L2NORM) != 0;
    const bool softplus = (p.flags & GDN_SOFTPLUS) != 0;
    const bool sigmoid = (p.flags & GDN_SIGMOID) != 0;
    const float rmul = (p.flags & GDN_NO_RETRIEVE) ? 0.0f : 1.0f;  // the retrieval term's weight
    const float a_mul = (!PREP && p.a && softplus) ? -expf(p.A_log[h]) : 0.0f;
    const float a_bias = (!PREP && p.a && softplus) ? p.dt_bias[h] : 0.0f;
    TS* outp = static_cast<TS*>(p.out);

    int captured = 0;  // tokens recorded (0 without capture)
    CaptureRow crow{};
    if (p.cap > 0) {
        captured = captured_tokens(p.counts, p.active, p.cap, b, end - start);
        crow = capture_row(p.capsule, b, p.cap, p.H, p.HQ, Kr, p.V);
    }
    const bool cap_g = vt == 0 && wave == 0 && lane == 0;
    const bool cap_k = vt == 0 && wave == 0 && grp == 0 && h == kh * p.G;
    const bool cap_d = gl < CPL && vbase + gl < p.V;
    // record slot i: g, the lane's share of k^ = kv * rk, and delta of column vbase + gl
    auto capture = [&](int i, float g, const float (&kv)[EPL], float rk, float dmine) {
        if (cap_g) *crow.g(i, h) = g;
        if (cap_k) {
            float* kd = crow.k(i, kh);
#pragma unroll
            for (int m = 0; m < EPL / 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (KX || 4 * (gl + LPC * m) + e < Kr) kd[4 * (gl + LPC * m) + e] = kv[4 * m + e] * rk;
        }
        if (cap_d) crow.d(i, h)[vbase + gl] = dmine;
    };
    auto capture_zeros = [&]() {
        for (int i = captured; i < p.cap; ++i) {
            if (cap_g) *crow.g(i, h) = 0.0f;
            if (cap_k) {
                float* kd = crow.k(i, kh);
#pragma unroll
                for (int m = 0; m < EPL / 4; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (KX || 4 * (gl + LPC * m) + e < Kr) kd[4 * (gl + LPC * m) + e] = 0.0f;
            }
            if (cap_d) crow.d(i, h)[vbase + gl] = 0.0f;
        }
    };

    if constexpr (SHORT) {
        // ---- 2 .. TSH tokens, a whole column tile and a carried state (block-uniform conditions) --
        constexpr int TSH = GDN_DECODE_SHORT;
        constexpr int BC = NW * WC;        // columns of the block
        constexpr int EPT = K / 32;        // q/k elements per staging thread (32 threads per token)
        __shared__ __align__(16) float shq[TSH][K];
        __shared__ __align__(16) float shk[TSH][K];
        __shared__ float shv[TSH][BC];
        __shared__ float shg[TSH], shb[TSH], shqk[TSH];
        __shared__ __align__(16) float shgk[PK ? TSH : 1][PK ? K : 1];  // PK: decays per key channel
        const int ntok = end - start;  // tokens of the sequence
        const bool full_tile = (vt * NW + NW) * WC <= p.V;
        if (ntok >= 2 && ntok <= TSH && full_tile && p.state_in != nullptr && p.state_out != nullptr) {
            const int tid = (int)threadIdx.x;
            const int vb0 = vt * NW * WC;  // first column of the block
            // the state tile first: its loads are in flight while the tokens are staged
            f32x4 sc[CPL][EPL / 4];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float* sp = p.state_in + (col0 + vbase + c) * Kr;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) sc[c][i] = ld_row4<KX, NT>(sp, 4 * (gl + LPC * i), Kr);
            }
            // (1) token operands, once per block: 32 threads per token, EPT elements each
            for (int tb = 0; tb < ntok; tb += 2 * NW) {
                const int t = tb + tid / 32, j = tid % 32;
                const bool live = t < ntok;
                const int tt = start + (live ? t : 0);
                float qv[EPT], kv[EPT];
                const int ej = j * EPT;  // first element of the thread's slice
                if constexpr (PREP) {
                    const float* qp = p.qk_prep + ((size_t)tt * p.HQ + kh) * Kr + ej;
                    const float* kp = p.qk_prep + (((size_t)p.N + tt) * p.HQ + kh) * Kr + ej;
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        qv[e] = (KX || ej + e < Kr) ? qp[e] : 0.0f;
                        kv[e] = (KX || ej + e < Kr) ? kp[e] : 0.0f;
                    }
                } else {
                    const TS* qp = static_cast<const TS*>(p.x.q) + (size_t)tt * p.x.sq + (size_t)kh * Kr + ej;
                    const TS* kp = static_cast<const TS*>(p.x.k) + (size_t)tt * p.x.sk + (size_t)kh * Kr + ej;
                    if constexpr (!KX) {
#pragma unroll
                        for (int e = 0; e < EPT; ++e) {
                            qv[e] = ej + e < Kr ? to_f32<T>(qp[e]) : 0.0f;
                            kv[e] = ej + e < Kr ? to_f32<T>(kp[e]) : 0.0f;
                        }
                    } else if constexpr (EPT % 4 == 0) {
#pragma unroll
                        for (int e = 0; e < EPT; e += 4) {
                            const f32x4 a4 = load4<T>(qp + e), b4 = load4<T>(kp + e);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                qv[e + i] = a4[i];
                                kv[e + i] = b4[i];
                            }
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < EPT; ++e) {
                            qv[e] = to_f32<T>(qp[e]);
                            kv[e] = to_f32<T>(kp[e]);
                        }
                    }
                }
                float qk = 0.0f, nq = 0.0f, nk = 0.0f;
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    qk = fmaf(qv[e], kv[e], qk);
                    nq = fmaf(qv[e], qv[e], nq);
                    nk = fmaf(kv[e], kv[e], nk);
                }
                qk = group_sum<32>(qk);
                float rq = 1.0f, rk = 1.0f;
                if (!PREP && l2) {
                    rq = rsqrtf(group_sum<32>(nq) + 1e-12f);
                    rk = rsqrtf(group_sum<32>(nk) + 1e-12f);
                }
                if (live) {
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        shq[t][j * EPT + e] = qv[e] * rq;
                        shk[t][j * EPT + e] = kv[e] * rk;
                    }
                    if constexpr (PK) {
                        const size_t gi = ((size_t)tt * p.H + h) * Kr + ej;
#pragma unroll
                        for (int e = 0; e < EPT; ++e) {
                            const float x = (KX || ej + e < Kr) ? load_any(p.a, p.gate_dtype, gi + e) : 0.0f;
                            shgk[t][j * EPT + e] = softplus ? expf(a_mul * softplus_f(x + a_bias)) : expf(x);
                        }
                    }
                    if (j == 0) {
                        float g, beta;
                        const size_t gi = (size_t)tt * p.H + h;
                        if constexpr (PREP) {
                            g = p.gb_prep[gi];
                            beta = p.gb_prep[(size_t)p.N * p.H + gi];
                        } else {
                            g = 1.0f;
                            if (!PK && p.a) {
                                const float x = load_any(p.a, p.gate_dtype, gi);
                                g = softplus ? expf(a_mul * softplus_f(x + a_bias)) : expf(x);
                            }
                            beta = 1.0f;
                            if (p.b) {
                                const float x = load_any(p.b, p.gate_dtype, gi);
                                beta = sigmoid ? 1.0f / (1.0f + expf(-x)) : x;
                            }
                        }
                        shg[t] = g;
                        shb[t] = beta;
                        shqk[t] = qk * rq * rk;
                    }
                }
            }
            for (int i = tid; i < ntok * BC; i += 64 * NW) {
                const int t = i / BC, col = i % BC;
                shv[t][col] = to_f32<T>(static_cast<const TS*>(p.x.v)[(size_t)(start + t) * p.x.sv + (size_t)h * p.V + vb0 + col]);
            }
            __syncthreads();

            // (2) the tile's columns go through the tokens together, the state kept as s = c * s' with
            // a block-uniform scale c (the product of the decays so far), so that a token's update is
            // one fused multiply-add per element.  When c would leave [1e-30, 1e30] (including a zero
            // decay) it is folded into s' first.
            const int lc = vbase - vb0;
            float cs = 1.0f;
#pragma unroll
            for (int t = 0; t < TSH; ++t) {
                if (t >= ntok) break;
                f32x4 qf[EPL / 4], kf[EPL / 4];
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) {
                    qf[i] = *reinterpret_cast<const f32x4*>(&shq[t][4 * (gl + LPC * i)]);
                    kf[i] = *reinterpret_cast<const f32x4*>(&shk[t][4 * (gl + LPC * i)]);
                }
                const float g = shg[t], beta = shb[t], qk = shqk[t];
                float cn = cs * g;
                if constexpr (PK) {
                    // per-key decays (g is 1): decay each channel of the resident tile directly
#pragma unroll
                    for (int i = 0; i < EPL / 4; ++i) {
                        const f32x4 gv = *reinterpret_cast<const f32x4*>(&shgk[t][4 * (gl + LPC * i)]);
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
#pragma unroll
                            for (int e = 0; e < 4; ++e) sc[c][i][e] *= gv[e];
                    }
                } else if (!(cn >= 1e-30f && cn <= 1e30f)) {
                    // block-uniform: fold the scale, this token's decay included, into the kept state
                    // (a zero or tiny decay leaves a zero state, as the recurrence does)
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
#pragma unroll
                        for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
                            for (int e = 0; e < 4; ++e) sc[c][i][e] *= cn;
                    cn = 1.0f;
                }
                cs = cn;
                const float icn = 1.0f / cn;
                float pk[CPL], pq[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    pk[c] = 0.0f;
                    pq[c] = 0.0f;
#pragma unroll
                    for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pk[c] = fmaf(sc[c][i][e], kf[i][e], pk[c]);
                            pq[c] = fmaf(sc[c][i][e], qf[i][e], pq[c]);
                        }
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    pk[c] = group_sum<LPC>(pk[c]);
                    pq[c] = group_sum<LPC>(pq[c]);
                }
                float mine = 0.0f, dm = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const float r = rmul * (cn * pk[c]);
                    const float delta = beta * (shv[t][lc + c] - r);
                    const float o = p.scale * fmaf(cn, pq[c], delta * qk);
                    const float dc = delta * icn;
#pragma unroll
                    for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sc[c][i][e] = fmaf(dc, kf[i][e], sc[c][i][e]);
                    if (gl == c) {
                        mine = o;
                        dm = delta;
                    }
                }
                if (gl < CPL) outp[((size_t)(start + t) * p.H + h) * p.V + vbase + gl] = from_f32<T>(mine);
                if (cap_d && t < captured) crow.d(t, h)[vbase + gl] = dm;
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float* sp = p.state_out + (col0 + vbase + c) * Kr;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) {
                    f32x4 v = sc[c][i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] *= cs;
                    st_row4<KX, NT>(sp, 4 * (gl + LPC * i), Kr, v);
                }
            }
            if (p.cap > 0) {
#pragma unroll
                for (int t = 0; t < TSH; ++t) {
                    if (t >= captured) break;
                    if (cap_g) *crow.g(t, h) = shg[t];
                    if (cap_k) {
                        float* kd = crow.k(t, kh);
#pragma unroll
                        for (int m = 0; m < EPL / 4; ++m)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (KX || 4 * (gl + LPC * m) + e < Kr)
                                    kd[4 * (gl + LPC * m) + e] = shk[t][4 * (gl + LPC * m) + e];
                    }
                }
                capture_zeros();
            }
            return;
        }
    }

    if constexpr (GDN_DECODE_STREAM > 0 && !SHORT) {
        // One token, a whole column tile and a carried state (block-uniform conditions): stream the
        // columns with GDN_DECODE_STREAM columns of loads ahead, storing each column as soon as it is
        // updated, so that each lane keeps few accesses in flight and reads and writes interleave.
        constexpr int PD = GDN_DECODE_STREAM < CPL ? GDN_DECODE_STREAM : CPL;
        const bool full_tile = (vt * NW + NW) * WC <= p.V;
        if (end - start == 1 && full_tile && p.state_in != nullptr && p.state_out != nullptr) {
            TokenOps<EPL, CPL, PK> tok;
            load_token<T, K, LPC, CPL, PREP, PK, KX>(p, start, h, kh, gl, vbase, tok);
            f32x4 ring[PD + 1][EPL / 4];
            auto load_col = [&](int c, f32x4 (&dst)[EPL / 4]) {
                const float* sp = p.state_in + (col0 + vbase + c) * Kr;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) dst[i] = ld_row4<KX, NT>(sp, 4 * (gl + LPC * i), Kr);
            };
#pragma unroll
            for (int c = 0; c < PD; ++c) load_col(c, ring[c]);
            float g, beta;
            if constexpr (PREP) {
                g = tok.ga;
                beta = tok.gb;
            } else {
                g = 1.0f;
                if (!PK && p.a) g = softplus ? expf(a_mul * softplus_f(tok.ga + a_bias)) : expf(tok.ga);
                beta = 1.0f;
                if (p.b) beta = sigmoid ? 1.0f / (1.0f + expf(-tok.gb)) : tok.gb;
            }
            float gk[PK ? EPL : 1];  // PK: the lane's channel decays (the state is decayed before the dots)
            if constexpr (PK) {
                if ((int)threadIdx.x < K)
                    gks[threadIdx.x] = softplus ? expf(a_mul * softplus_f(tok.gkr + a_bias)) : expf(tok.gkr);
                __syncthreads();
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) {
                    const f32x4 gv = *reinterpret_cast<const f32x4*>(&gks[4 * (gl + LPC * i)]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) gk[4 * i + e] = gv[e];
                }
            }
            float qk = 0.0f, nq = 0.0f, nk = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                qk = fmaf(tok.q[e], tok.k[e], qk);
                if constexpr (!PREP) {
                    nq = fmaf(tok.q[e], tok.q[e], nq);
                    nk = fmaf(tok.k[e], tok.k[e], nk);
                }
            }
            qk = group_sum<LPC>(qk);
            float rq = 1.0f, rk = 1.0f;
            if constexpr (!PREP) {
                if (l2) {
                    rq = rsqrtf(group_sum<LPC>(nq) + 1e-12f);
                    rk = rsqrtf(group_sum<LPC>(nk) + 1e-12f);
                }
            }
            const float oscale = p.scale * rq;
            float mine = 0.0f, dmine = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if (c + PD < CPL) load_col(c + PD, ring[(c + PD) % (PD + 1)]);
                f32x4(&sc)[EPL / 4] = ring[c % (PD + 1)];
                if constexpr (PK) {
#pragma unroll
                    for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sc[i][e] *= gk[4 * i + e];
                }
                float pk = 0.0f, pq = 0.0f;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pk = fmaf(sc[i][e], tok.k[4 * i + e], pk);
                        pq = fmaf(sc[i][e], tok.q[4 * i + e], pq);
                    }
                pk = group_sum<LPC>(pk);
                pq = group_sum<LPC>(pq);
                const float r = rmul * (g * rk * pk);
                const float delta = beta * (tok.v[c] - r);
                const float dk = delta * rk;
                const float o = oscale * fmaf(g, pq, dk * qk);
                float* sp = p.state_out + (col0 + vbase + c) * Kr;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) {
                    f32x4 nv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) nv[e] = fmaf(dk, tok.k[4 * i + e], PK ? sc[i][e] : g * sc[i][e]);
                    st_row4<KX, NT>(sp, 4 * (gl + LPC * i), Kr, nv);
                }
                if (gl == c) {
                    mine = o;
                    dmine = delta;
                }
            }
            if (gl < CPL) outp[((size_t)start * p.H + h) * p.V + vbase + gl] = from_f32<T>(mine);
            if (p.cap > 0) {
                if (captured > 0) capture(0, g, tok.k, rk, dmine);
                capture_zeros();
            }
            return;
        }
    }

    float s[CPL][EPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const bool valid = (vbase + c < p.V) && p.state_in != nullptr;
        const float* sp = p.state_in + (col0 + vbase + c) * Kr;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
            const f32x4 v = valid ? ld_row4<KX, NT>(sp, 4 * (gl + LPC * i), Kr) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) s[c][4 * i + e] = v[e];
        }
    }

    TokenOps<EPL, CPL, PK> cur;
    if (start < end) load_token<T, K, LPC, CPL, PREP, PK, KX>(p, start, h, kh, gl, vbase, cur);
    for (int t = start; t < end; ++t) {
        TokenOps<EPL, CPL, PK> nxt;
        if (t + 1 < end) load_token<T, K, LPC, CPL, PREP, PK, KX>(p, t + 1, h, kh, gl, vbase, nxt);

        float g, beta;
        if constexpr (PREP) {
            g = cur.ga;
            beta = cur.gb;
        } else {
            g = 1.0f;
            if (!PK && p.a) g = softplus ? expf(a_mul * softplus_f(cur.ga + a_bias)) : expf(cur.ga);
            beta = 1.0f;
            if (p.b) beta = sigmoid ? 1.0f / (1.0f + expf(-cur.gb)) : cur.gb;
        }
        if constexpr (PK) {
            // decay the lane's state slice channel by channel (decays staged once per block); g
            // stays 1 below.  The loop is block-uniform, so every thread reaches both barriers.
            __syncthreads();  // the previous token's decays have been read
            if ((int)threadIdx.x < K)
                gks[threadIdx.x] = softplus ? expf(a_mul * softplus_f(cur.gkr + a_bias)) : expf(cur.gkr);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i) {
                const f32x4 gv = *reinterpret_cast<const f32x4*>(&gks[4 * (gl + LPC * i)]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) s[c][4 * i + e] *= gv[e];
            }
        }

        float pk[CPL], pq[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            pk[c] = 0.0f;
            pq[c] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                pk[c] = fmaf(s[c][e], cur.k[e], pk[c]);
                pq[c] = fmaf(s[c][e], cur.q[e], pq[c]);
            }
        }
        float qk = 0.0f, nq = 0.0f, nk = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qk = fmaf(cur.q[e], cur.k[e], qk);
            if constexpr (!PREP) {
                nq = fmaf(cur.q[e], cur.q[e], nq);
                nk = fmaf(cur.k[e], cur.k[e], nk);
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            pk[c] = group_sum<LPC>(pk[c]);
            pq[c] = group_sum<LPC>(pq[c]);
        }
        qk = group_sum<LPC>(qk);
        float rq = 1.0f, rk = 1.0f;
        if constexpr (!PREP) {
            if (l2) {
                rq = rsqrtf(group_sum<LPC>(nq) + 1e-12f);
                rk = rsqrtf(group_sum<LPC>(nk) + 1e-12f);
            }
        }
        const float oscale = p.scale * rq;
        float mine = 0.0f, dmine = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float r = rmul * (g * rk * pk[c]);
            const float delta = beta * (cur.v[c] - r);
            const float dk = delta * rk;  // coefficient of the raw k
            const float o = oscale * fmaf(g, pq[c], dk * qk);
#pragma unroll
            for (int e = 0; e < EPL; ++e) s[c][e] = fmaf(dk, cur.k[e], PK ? s[c][e] : g * s[c][e]);
            if (gl == c) {
                mine = o;
                dmine = delta;
            }
        }
        if (gl < CPL && vbase + gl < p.V) outp[((size_t)t * p.H + h) * p.V + vbase + gl] = from_f32<T>(mine);
        if (t - start < captured) capture(t - start, g, cur.k, rk, dmine);
        cur = nxt;
    }

    if (p.state_out != nullptr) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (vbase + c >= p.V) continue;
            float* sp = p.state_out + (col0 + vbase + c) * Kr;
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i)
                st_row4<KX, NT>(sp, 4 * (gl + LPC * i), Kr,
                                f32x4{s[c][4 * i], s[c][4 * i + 1], s[c][4 * i + 2], s[c][4 * i + 3]});
        }
    }
    if (p.cap > 0) capture_zeros();
}

template <typename T, int K, int LPC, int CPL, int NW, bool PREP, bool NT, bool PK, bool SHORT, bool KX>
hipError_t launch_tile(ScanArgs p, hipStream_t stream) {
    constexpr int BC = (64 / LPC) * CPL * NW;  // columns per block
    p.n_vtiles = (p.V + BC - 1) / BC;
    const long long blocks = (long long)p.B * p.H * p.n_vtiles;
    if (blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    p.n_blocks = (int)blocks;
    hipLaunchKernelGGL((scan_kernel<T, K, LPC, CPL, NW, PREP, NT, PK, SHORT, KX>), dim3((unsigned)blocks), dim3(64 * NW), 0,
                       stream, p);
    return hipGetLastError();
}

// DECODE tile: 16-lane groups (8 for K = 32), GDN_DECODE_CPL columns per group (half that at
// K = 256), GDN_DECODE_NW waves per block.  The state is streamed once, with non-temporal accesses.
#ifndef GDN_DECODE_CPL
#define GDN_DECODE_CPL 4
#endif
#ifndef GDN_DECODE_NW
#define GDN_DECODE_NW 4
#endif
template <typename T, int K, bool PREP, bool PK, bool KX>
hipError_t launch_k(const ScanArgs& p, hipStream_t stream) {
    constexpr int LPC = K >= 64 ? 16 : 8;
    constexpr int CPL = K >= 256 ? (GDN_DECODE_CPL > 1 ? GDN_DECODE_CPL / 2 : 1) : GDN_DECODE_CPL;
    // calls with more tokens than sequences hold short sequences: SHORT instances
    if (p.N > p.B) return launch_tile<T, K, LPC, CPL, GDN_DECODE_NW, PREP, true, PK, true, KX>(p, stream);
    return launch_tile<T, K, LPC, CPL, GDN_DECODE_NW, PREP, true, PK, false, KX>(p, stream);
}

// Key widths 32, 64, 128 and 256 run exactly; any other width up to 256 runs on the next of them
// with the lanes' elements past K zero (element-wise row accesses).
template <typename T, bool PREP, bool PK>
hipError_t launch_t(const ScanArgs& p, hipStream_t stream) {
    switch (p.K) {
        case 32: return launch_k<T, 32, PREP, PK, true>(p, stream);
        case 64: return launch_k<T, 64, PREP, PK, true>(p, stream);
        case 128: return launch_k<T, 128, PREP, PK, true>(p, stream);
        case 256: return launch_k<T, 256, PREP, PK, true>(p, stream);
        default: break;
    }
    if (p.K < 1 || p.K > 256) return hipErrorInvalidValue;
    switch (padded_key_width(p.K)) {
        case 32: return launch_k<T, 32, PREP, PK, false>(p, stream);
        case 64: return launch_k<T, 64, PREP, PK, false>(p, stream);
        case 128: return launch_k<T, 128, PREP, PK, false>(p, stream);
        default: return launch_k<T, 256, PREP, PK, false>(p, stream);
    }
}

template <bool PREP, bool PK>
hipError_t launch_p(const ScanArgs& p, int dtype, hipStream_t stream) {
    switch (dtype) {
        case GDN_F32: return launch_t<F32, PREP, PK>(p, stream);
        case GDN_BF16: return launch_t<BF16, PREP, PK>(p, stream);
        case GDN_F16: return launch_t<F16, PREP, PK>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_decode(const ScanLaunch& a, hipStream_t stream) {
    ScanArgs p;
    p.x = a.x;
    p.qk_prep = a.qk_prep;
    p.gb_prep = a.gb_prep;
    p.a = a.a;
    p.b = a.b;
    p.A_log = a.A_log;
    p.dt_bias = a.dt_bias;
    p.state_in = a.state_in;
    p.out = a.out;
    p.state_out = a.state_out;
    p.offsets = a.offsets;
    p.dev_status = a.dev_status;
    p.B = a.B;
    p.N = a.N;
    p.HQ = a.HQ;
    p.H = a.H;
    p.K = a.K;
    p.V = a.V;
    p.G = a.H / a.HQ;
    p.gate_dtype = a.gate_dtype;
    p.flags = a.flags;
    p.scale = a.scale;
    p.n_vtiles = 0;
    p.n_blocks = 0;
    p.cap = a.cap;
    p.counts = a.counts;
    p.active = a.active;
    p.capsule = a.capsule;
    if (a.qk_prep != nullptr) return launch_p<true, false>(p, a.qkv_dtype, stream);
    if ((a.flags & GDN_GATE_PER_KEY) && a.a != nullptr) return launch_p<false, true>(p, a.qkv_dtype, stream);
    return launch_p<false, false>(p, a.qkv_dtype, stream);
}

}  // namespace gdn
