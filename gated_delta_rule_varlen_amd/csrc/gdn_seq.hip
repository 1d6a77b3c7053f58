// gdn_seq.hip -- gated delta-rule recurrence, SEQ path: token-sequential form with the state
// resident in VGPRs for a whole sequence and the token operands staged through LDS (gfx950).
//
// Operation: paged_ssm.rs page, kernel string DELTA (see gdn.h).  A block owns one (sequence, value
// head) and NW column tiles of it, one per wave; a column's K-vector state is split over a group of
// LPC lanes exactly as in the DECODE kernel (16-byte chunks, DPP group reductions).  What differs
// is how the per-token operands arrive:
//
//   * the sequence is walked in chunks of TC tokens.  For each chunk the whole block cooperatively
//     loads the raw q/k rows of the key head, the decay/rate inputs and the block's v columns with
//     16-byte loads, normalises q and k (DPP reductions over K/VEC-lane groups), evaluates the gates
//     and q^.k^ once per token, and writes fp32 operands to LDS -- instead of every wave redoing the
//     norms, the transcendental gate math and the latency-bound global loads for every token;
//   * staging is double-buffered through registers: the global loads of chunk c+1 are issued before
//     the recurrence walks chunk c out of LDS, so their latency hides behind TC tokens of work;
//   * each token then costs, per lane and column, EPL fused multiply-adds for each of k.s and q.s,
//     one 4-step DPP reduction pair and EPL multiply-adds for the update
//         r = g (k^.s),  delta = beta (v - r),  out = scale (g (q^.s) + delta (q^.k^)),
//         s <- g s + delta k^;
//   * outputs of a chunk are collected in LDS and written back as 16-byte vectors;
//   * key widths other than 32, 64, 128 and 256 run on the next compiled width with the elements
//     past K zero (element-wise q/k and state accesses; "KX = false" instances);
//   * blocks take the sequences longest first (ranked in-block by length, for up to 64 sequences);
//   * with a per-key-channel decay (GDN_GATE_PER_KEY; "PK" instances) the staging also evaluates
//     the decay of every (token, key channel) once per block into LDS, and the recurrence decays
//     each state slice channel by channel before the dot products;
//   * with capture (speculative decoding: paged_ssm.rs page, DELTA_CAPTURE_INIT / _STEP) the first
//     captured tokens of a sequence also record g and k^ (copied out of the LDS stage by the head's
//     first block; k^ only for the first value head of each key head) and delta (by the lane that
//     produces the column's output); the slots after them are zeroed.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

struct SeqArgs {
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
    int n_vtiles;
    int n_blocks;
    int vec_ok;  // V is a multiple of the 16-byte vector width: v columns and outputs move as vectors
    int cap;                // capture slots per sequence (0 = no capture)
    const int32_t* counts;  // [B]
    const int32_t* active;  // [1] or NULL
    float* capsule;         // [B, cap*(H + HQ*K + H*V)]
};

template <typename T, int K, int LPC, int CPL, int NW, bool PREP, bool PK>
struct Cfg {
    using TS = typename T::storage;
    static constexpr int NT = 64 * NW;                                  // threads per block
    static constexpr int EPL = K / LPC;                                 // state elements per lane
    static constexpr int WC = (64 / LPC) * CPL;                         // columns per wave
    static constexpr int BC = NW * WC;                                  // columns per block
    // tokens per chunk; halved with per-key decays, whose LDS stage would otherwise cost a block per CU
    static constexpr int TC = (PK ? 1024 : 2048) / K;
    static constexpr int SVEC = PREP ? 4 : 16 / (int)sizeof(TS);        // q/k elements per 16-byte load
    static constexpr int RL = K / SVEC;                                 // lanes per token for q/k staging
    static constexpr int TPP = NT / RL;                                 // tokens per staging pass
    static constexpr int PASSES = (TC + TPP - 1) / TPP;
    static constexpr int VVEC = 16 / (int)sizeof(TS);                   // v / out elements per 16 bytes
    static constexpr int VPT = BC / VVEC;                               // v vectors per token
    static constexpr int VPASSES = (TC * VPT + NT - 1) / NT;
    static_assert(EPL % 4 == 0 && RL <= 64 && (RL & (RL - 1)) == 0 && BC % VVEC == 0, "tile shape");
};

// Raw operands of one chunk as fetched by one thread (kept in registers across a chunk of work).
template <int PASSES, int VPASSES, int GKN>
struct Fetch {
    u32x4 q[PASSES];
    u32x4 k[PASSES];
    u32x4 v[VPASSES];
    float ga, gb;
    float gk[GKN];  // per-key decay inputs of the thread's q/k elements (PK only)
};

constexpr int kRankedSeqs = 64;  // sequences ranked by length in-block (more keep their order)

template <typename T, int K, int LPC, int CPL, int NW, bool PREP, bool PK, bool KX>
__global__ __launch_bounds__(64 * NW) void seq_kernel(SeqArgs p) {
    static_assert(!(PK && PREP), "the per-key decay is evaluated in-kernel from raw inputs");
    // K is the compiled key width; rows are Kr wide (Kr < K: the elements past Kr are zero)
    const int Kr = KX ? K : p.K;
    using C_ = Cfg<T, K, LPC, CPL, NW, PREP, PK>;
    using TS = typename C_::TS;
    constexpr int EPL = C_::EPL, WC = C_::WC, BC = C_::BC, TC = C_::TC;
    constexpr int SVEC = C_::SVEC, RL = C_::RL, TPP = C_::TPP, PASSES = C_::PASSES;
    constexpr int VVEC = C_::VVEC, VPT = C_::VPT, VPASSES = C_::VPASSES, NT = C_::NT;

    __shared__ __align__(16) float sq[2][TC][K];
    __shared__ __align__(16) float sk[2][TC][K];
    __shared__ __align__(16) float sv[2][TC][BC];
    __shared__ float sg[2][TC], sb[2][TC], sqk[2][TC];
    __shared__ __align__(16) float so[TC][BC];
    __shared__ __align__(16) float sgk[PK ? 2 : 1][PK ? TC : 1][PK ? K : 1];
    constexpr int GKN = PK ? PASSES * SVEC : 1;

    const bool malformed = offsets_malformed(p.offsets, p.B, p.N);
    report_status(p.dev_status, malformed);
    if (malformed) return;

    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, p.G * p.n_vtiles);
    const int vt = blk % p.n_vtiles;
    const int bh = blk / p.n_vtiles;
    const int h = bh % p.H;
    const int tid = (int)threadIdx.x;
    // Blocks live as long as their sequence and can outnumber the resident ones, so the sequences are
    // taken longest first (list scheduling): with up to kRankedSeqs sequences every block ranks
    // the lengths in LDS and serves the sequence whose rank is its logical index.
    int b = bh / p.H;
    if (p.B <= kRankedSeqs) {
        __shared__ int s_len[kRankedSeqs];
        __shared__ int s_pick;
        for (int i = tid; i < p.B; i += NT) s_len[i] = p.offsets[i + 1] - p.offsets[i];
        __syncthreads();
        const int want = b;
        for (int i = tid; i < p.B; i += NT) {
            const int li = s_len[i];
            int rank = 0;
            for (int j = 0; j < p.B; ++j) rank += (s_len[j] > li) || (s_len[j] == li && j < i);
            if (rank == want) s_pick = i;
        }
        __syncthreads();
        b = s_pick;
    }
    const int kh = h / p.G;
    const int wave = tid / 64, lane = tid % 64;
    const int grp = lane / LPC, gl = lane % LPC;
    const int cw = wave * WC + grp * CPL;  // first block-local column of this lane group
    const int v0 = vt * BC;                // first value column of the block
    const size_t col0 = ((size_t)b * p.H + h) * p.V;

    float s[CPL][EPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const bool valid = (v0 + cw + c < p.V) && p.state_in != nullptr;
        const float* sp = p.state_in + (col0 + v0 + cw + c) * Kr;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
            const f32x4 v = valid ? ld_row4<KX, false>(sp, 4 * (gl + LPC * i), Kr) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) s[c][4 * i + e] = v[e];
        }
    }

    const int start = p.offsets[b], end = p.offsets[b + 1];
    const int nchunks = (end - start + TC - 1) / TC;
    const bool l2 = (p.flags & GDN_L2NORM) != 0;
    const bool softplus = (p.flags & GDN_SOFTPLUS) != 0;
    const bool sigmoid = (p.flags & GDN_SIGMOID) != 0;
    const float rmul = (p.flags & GDN_NO_RETRIEVE) ? 0.0f : 1.0f;  // the retrieval term's weight
    const float a_mul = (!PREP && p.a && softplus) ? -expf(p.A_log[h]) : 0.0f;
    const float a_bias = (!PREP && p.a && softplus) ? p.dt_bias[h] : 0.0f;
    const TS* const xq = static_cast<const TS*>(p.x.q);
    const TS* const xk = static_cast<const TS*>(p.x.k);
    const TS* const xv = static_cast<const TS*>(p.x.v);
    TS* outp = static_cast<TS*>(p.out);

    int captured = 0;  // tokens recorded (0 without capture)
    CaptureRow crow{};
    if (p.cap > 0) {
        captured = captured_tokens(p.counts, p.active, p.cap, b, end - start);
        crow = capture_row(p.capsule, b, p.cap, p.H, p.HQ, Kr, p.V);
    }
    const bool cap_d = gl < CPL && v0 + cw + gl < p.V;  // this lane records delta of its output column

    // ---- staging: global -> registers (fetch) and registers -> LDS (commit) ------------------------
    auto fetch = [&](int t0, int n, Fetch<PASSES, VPASSES, GKN>& f) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int ti = ps * TPP + tid / RL, rl = tid % RL;
            f.q[ps] = f.k[ps] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (PK) {
#pragma unroll
                for (int e = 0; e < SVEC; ++e) f.gk[ps * SVEC + e] = 0.0f;
                if (ti < n && ti < TC) {
                    const size_t gi = ((size_t)(t0 + ti) * p.H + h) * Kr + rl * SVEC;
                    if constexpr (KX) {
#pragma unroll
                        for (int e = 0; e < SVEC; e += 4) {
                            const f32x4 av = load4_gate<T>(p.a, p.gate_dtype, gi + e);
#pragma unroll
                            for (int j = 0; j < 4; ++j) f.gk[ps * SVEC + e + j] = av[j];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < SVEC; ++e)
                            if (rl * SVEC + e < Kr) f.gk[ps * SVEC + e] = load_any(p.a, p.gate_dtype, gi + e);
                    }
                }
            }
            if (ti < n) {
                const size_t t = (size_t)(t0 + ti);
                if constexpr (PREP) {
                    f.q[ps] = ld_raw16<float, 4, KX>(p.qk_prep + (t * p.HQ + kh) * Kr, rl * SVEC, Kr);
                    f.k[ps] = ld_raw16<float, 4, KX>(p.qk_prep + (((size_t)p.N + t) * p.HQ + kh) * Kr, rl * SVEC, Kr);
                } else {
                    f.q[ps] = ld_raw16<TS, SVEC, KX>(xq + t * p.x.sq + (size_t)kh * Kr, rl * SVEC, Kr);
                    f.k[ps] = ld_raw16<TS, SVEC, KX>(xk + t * p.x.sk + (size_t)kh * Kr, rl * SVEC, Kr);
                }
            }
        }
        f.ga = f.gb = 0.0f;
        if (tid < n) {
            const size_t gi = (size_t)(t0 + tid) * p.H + h;
            if constexpr (PREP) {
                f.ga = p.gb_prep[gi];
                f.gb = p.gb_prep[(size_t)p.N * p.H + gi];
            } else {
                if (!PK && p.a) f.ga = load_any(p.a, p.gate_dtype, gi);
                if (p.b) f.gb = load_any(p.b, p.gate_dtype, gi);
            }
        }
#pragma unroll
        for (int vp = 0; vp < VPASSES; ++vp) {
            const int idx = vp * NT + tid;
            const int ti = idx / VPT, j = idx % VPT;
            const int col = v0 + j * VVEC;
            f.v[vp] = u32x4{0u, 0u, 0u, 0u};
            if (idx < TC * VPT && ti < n) {
                const TS* src = xv + (size_t)(t0 + ti) * p.x.sv + (size_t)h * p.V + col;
                if (p.vec_ok && col + VVEC <= p.V) {
                    f.v[vp] = *reinterpret_cast<const u32x4*>(src);
                } else {
                    union {
                        u32x4 v;
                        TS e[VVEC];
                    } u;
                    u.v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < VVEC; ++e)
                        if (col + e < p.V) u.e[e] = src[e];
                    f.v[vp] = u.v;
                }
            }
        }
    };

    auto commit = [&](const Fetch<PASSES, VPASSES, GKN>& f, int buf) {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int ti = ps * TPP + tid / RL, rl = tid % RL;
            float qf[SVEC], kf[SVEC];
            if constexpr (PREP || std::is_same<T, F32>::value) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qf[e] = __uint_as_float(f.q[ps][e]);
                    kf[e] = __uint_as_float(f.k[ps][e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qf[2 * e] = to_f32<T>((uint16_t)(f.q[ps][e] & 0xffffu));
                    qf[2 * e + 1] = to_f32<T>((uint16_t)(f.q[ps][e] >> 16));
                    kf[2 * e] = to_f32<T>((uint16_t)(f.k[ps][e] & 0xffffu));
                    kf[2 * e + 1] = to_f32<T>((uint16_t)(f.k[ps][e] >> 16));
                }
            }
            float qk = 0.0f, nq = 0.0f, nk = 0.0f;
#pragma unroll
            for (int e = 0; e < SVEC; ++e) {
                qk = fmaf(qf[e], kf[e], qk);
                if constexpr (!PREP) {
                    nq = fmaf(qf[e], qf[e], nq);
                    nk = fmaf(kf[e], kf[e], nk);
                }
            }
            qk = group_sum<RL>(qk);
            float rq = 1.0f, rk = 1.0f;
            if constexpr (!PREP) {
                nq = group_sum<RL>(nq);
                nk = group_sum<RL>(nk);
                if (l2) {
                    rq = rsqrtf(nq + 1e-12f);
                    rk = rsqrtf(nk + 1e-12f);
                }
            }
            if (ti < TC) {
                float* dq = &sq[buf][ti][rl * SVEC];
                float* dk = &sk[buf][ti][rl * SVEC];
#pragma unroll
                for (int e = 0; e < SVEC; e += 4) {
                    *reinterpret_cast<f32x4*>(dq + e) = f32x4{qf[e] * rq, qf[e + 1] * rq, qf[e + 2] * rq, qf[e + 3] * rq};
                    *reinterpret_cast<f32x4*>(dk + e) = f32x4{kf[e] * rk, kf[e + 1] * rk, kf[e + 2] * rk, kf[e + 3] * rk};
                }
                if (rl == 0) sqk[buf][ti] = qk * rq * rk;
                if constexpr (PK) {
                    float* dg = &sgk[buf][ti][rl * SVEC];
#pragma unroll
                    for (int e = 0; e < SVEC; ++e) {
                        const float x = f.gk[ps * SVEC + e];
                        dg[e] = softplus ? expf(a_mul * softplus_f(x + a_bias)) : expf(x);
                    }
                }
            }
        }
        if (tid < TC) {
            float g, beta;
            if constexpr (PREP) {
                g = f.ga;
                beta = f.gb;
            } else {
                g = 1.0f;
                if (!PK && p.a) g = softplus ? expf(a_mul * softplus_f(f.ga + a_bias)) : expf(f.ga);
                beta = 1.0f;
                if (p.b) beta = sigmoid ? 1.0f / (1.0f + expf(-f.gb)) : f.gb;
            }
            sg[buf][tid] = g;
            sb[buf][tid] = beta;
        }
#pragma unroll
        for (int vp = 0; vp < VPASSES; ++vp) {
            const int idx = vp * NT + tid;
            const int ti = idx / VPT, j = idx % VPT;
            if (idx < TC * VPT) {
                float* dv = &sv[buf][ti][j * VVEC];
                if constexpr (std::is_same<T, F32>::value) {
                    *reinterpret_cast<f32x4*>(dv) = f32x4{__uint_as_float(f.v[vp][0]), __uint_as_float(f.v[vp][1]),
                                                          __uint_as_float(f.v[vp][2]), __uint_as_float(f.v[vp][3])};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dv[2 * e] = to_f32<T>((uint16_t)(f.v[vp][e] & 0xffffu));
                        dv[2 * e + 1] = to_f32<T>((uint16_t)(f.v[vp][e] >> 16));
                    }
                }
            }
        }
    };

    if (nchunks > 0) {
        Fetch<PASSES, VPASSES, GKN> f;
        fetch(start, min(TC, end - start), f);
        commit(f, 0);
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const int buf = c & 1;
            const int t0 = start + c * TC;
            const int n = min(TC, end - t0);
            const bool more = c + 1 < nchunks;
            if (more) fetch(t0 + TC, min(TC, end - t0 - TC), f);

            if (t0 - start < captured && vt == 0) {
                // g and k^ of the chunk's recorded tokens, straight from the LDS stage
                const int nc = min(n, captured - (t0 - start));
                for (int idx = tid; idx < nc; idx += NT) *crow.g(t0 - start + idx, h) = sg[buf][idx];
                if (h == kh * p.G)
                    for (int idx = tid; idx < nc * Kr; idx += NT)
                        crow.k(t0 - start + idx / Kr, kh)[idx % Kr] = sk[buf][idx / Kr][idx % Kr];
            }
            for (int i = 0; i < n; ++i) {
                float q[EPL], k[EPL];
#pragma unroll
                for (int m = 0; m < EPL / 4; ++m) {
                    const f32x4 qv = *reinterpret_cast<const f32x4*>(&sq[buf][i][4 * (gl + LPC * m)]);
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(&sk[buf][i][4 * (gl + LPC * m)]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        q[4 * m + e] = qv[e];
                        k[4 * m + e] = kv[e];
                    }
                }
                const float g = sg[buf][i], beta = sb[buf][i], qk = sqk[buf][i];
                if constexpr (PK) {
                    // channel-wise decay of the lane's state slice (g is 1 for PK)
#pragma unroll
                    for (int m = 0; m < EPL / 4; ++m) {
                        const f32x4 gv = *reinterpret_cast<const f32x4*>(&sgk[buf][i][4 * (gl + LPC * m)]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
#pragma unroll
                            for (int cc = 0; cc < CPL; ++cc) s[cc][4 * m + e] *= gv[e];
                    }
                }
                float pk[CPL], pq[CPL];
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    pk[cc] = 0.0f;
                    pq[cc] = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        pk[cc] = fmaf(s[cc][e], k[e], pk[cc]);
                        pq[cc] = fmaf(s[cc][e], q[e], pq[cc]);
                    }
                }
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    pk[cc] = group_sum<LPC>(pk[cc]);
                    pq[cc] = group_sum<LPC>(pq[cc]);
                }
                float mine = 0.0f, dmine = 0.0f;
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float d = beta * (sv[buf][i][cw + cc] - rmul * (g * pk[cc]));
                    const float o = p.scale * fmaf(g, pq[cc], d * qk);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) s[cc][e] = fmaf(d, k[e], PK ? s[cc][e] : g * s[cc][e]);
                    if (gl == cc) {
                        mine = o;
                        dmine = d;
                    }
                }
                if (gl < CPL) so[i][cw + gl] = mine;
                if (cap_d && t0 + i - start < captured) crow.d(t0 + i - start, h)[v0 + cw + gl] = dmine;
            }
            __syncthreads();  // outputs of the chunk are complete in LDS
            for (int idx = tid; idx < n * VPT; idx += NT) {
                const int ti = idx / VPT, j = idx % VPT;
                const int col = v0 + j * VVEC;
                TS* dst = outp + ((size_t)(t0 + ti) * p.H + h) * p.V + col;
                union {
                    u32x4 v;
                    TS e[VVEC];
                } u;
#pragma unroll
                for (int e = 0; e < VVEC; ++e) u.e[e] = from_f32<T>(so[ti][j * VVEC + e]);
                if (p.vec_ok && col + VVEC <= p.V) {
                    *reinterpret_cast<u32x4*>(dst) = u.v;
                } else {
#pragma unroll
                    for (int e = 0; e < VVEC; ++e)
                        if (col + e < p.V) dst[e] = u.e[e];
                }
            }
            if (more) commit(f, buf ^ 1);
            __syncthreads();  // next chunk staged; output buffer free again
        }
    }

    if (p.state_out != nullptr) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (v0 + cw + c >= p.V) continue;
            float* sp = p.state_out + (col0 + v0 + cw + c) * Kr;
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i)
                st_row4<KX, false>(sp, 4 * (gl + LPC * i), Kr,
                                   f32x4{s[c][4 * i], s[c][4 * i + 1], s[c][4 * i + 2], s[c][4 * i + 3]});
        }
    }

    if (p.cap > 0) {
        // zeros in the slots after the recorded tokens: g and k^ by the head's first block, delta
        // for the block's own columns
        for (int i = captured; i < p.cap; ++i) {
            if (vt == 0) {
                if (tid == 0) *crow.g(i, h) = 0.0f;
                if (h == kh * p.G)
                    for (int j = tid; j < Kr; j += NT) crow.k(i, kh)[j] = 0.0f;
            }
            for (int j = tid; j < BC; j += NT)
                if (v0 + j < p.V) crow.d(i, h)[v0 + j] = 0.0f;
        }
    }
}

template <typename T, int K, int LPC, int CPL, bool PREP, bool PK, bool KX>
hipError_t launch_tile(SeqArgs p, hipStream_t stream) {
    constexpr int NW = 4;
    using C_ = Cfg<T, K, LPC, CPL, NW, PREP, PK>;
    p.n_vtiles = (p.V + C_::BC - 1) / C_::BC;
    const long long blocks = (long long)p.B * p.H * p.n_vtiles;
    if (blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    p.n_blocks = (int)blocks;
    p.vec_ok = (p.V % C_::VVEC) == 0;
    hipLaunchKernelGGL((seq_kernel<T, K, LPC, CPL, NW, PREP, PK, KX>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

// Tile choice: two columns per lane group when that still gives 4 blocks per CU, else one; for
// K >= 128 and very few columns, 32-lane groups halve the columns per block once more.
template <typename T, int K, bool PREP, bool PK, bool KX>
hipError_t launch_k(const SeqArgs& p, hipStream_t stream) {
    constexpr int LPC = K >= 64 ? 16 : 8;
    constexpr int BC2 = 4 * (64 / LPC) * 2;
    const long long bh = (long long)p.B * p.H;
    if (bh * ((p.V + BC2 - 1) / BC2) >= 1024) return launch_tile<T, K, LPC, 2, PREP, PK, KX>(p, stream);
    if constexpr (K >= 128) {
        constexpr int BC1 = 4 * (64 / LPC);
        if (bh * ((p.V + BC1 - 1) / BC1) < 1024) return launch_tile<T, K, 32, 1, PREP, PK, KX>(p, stream);
    }
    return launch_tile<T, K, LPC, 1, PREP, PK, KX>(p, stream);
}

// Key widths 32, 64, 128 and 256 run exactly; any other width up to 256 runs on the next of them
// with the elements past K zero (element-wise row accesses).
template <typename T, bool PREP, bool PK>
hipError_t launch_t(const SeqArgs& p, hipStream_t stream) {
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
hipError_t launch_p(const SeqArgs& p, int dtype, hipStream_t stream) {
    switch (dtype) {
        case GDN_F32: return launch_t<F32, PREP, PK>(p, stream);
        case GDN_BF16: return launch_t<BF16, PREP, PK>(p, stream);
        case GDN_F16: return launch_t<F16, PREP, PK>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_seq(const ScanLaunch& a, hipStream_t stream) {
    SeqArgs p;
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
    p.vec_ok = 0;
    p.cap = a.cap;
    p.counts = a.counts;
    p.active = a.active;
    p.capsule = a.capsule;
    if (a.qk_prep != nullptr) return launch_p<true, false>(p, a.qkv_dtype, stream);
    if ((a.flags & GDN_GATE_PER_KEY) && a.a != nullptr) return launch_p<false, true>(p, a.qkv_dtype, stream);
    return launch_p<false, false>(p, a.qkv_dtype, stream);
}

}  // namespace gdn
