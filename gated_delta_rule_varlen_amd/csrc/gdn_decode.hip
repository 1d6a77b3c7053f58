// gdn_decode.hip -- one launch for a whole decode step: the varlen causal conv1d of each sequence's
// single token, the q/k norms and gates, and the gated delta-rule state update (gfx950, wave64).
//
// Operation: paged_ssm.rs page, kernel strings CONV and DELTA run back to back (the conv output is
// the recurrence's packed qkv row); the rate-activation page names launches per decode step as the
// cost of this layer type, which is what a single launch removes.  Every sequence holds 0 or 1
// tokens.  Results are bit-identical to gdn_conv1d_varlen followed by gdn_scan_varlen on its DECODE
// path: the conv arithmetic (bias, then taps in order, fp32 fma, the same SiLU) and its rounding to
// the I/O type are the same, and so is the recurrence code.
//
// A block owns (sequence b, key head kh): the q/k channels of kh and every value column of the G
// value heads that read kh, so that each carried window entry has exactly one reader and one
// writer (the q/k windows are shared by the G heads; with an in-place window, a split over blocks
// would race).  Two phases:
//   conv   each 4-channel group (q and k of kh, v of its heads) is computed by one thread; the
//          results, rounded to the I/O type, go to LDS; the thread then writes the new window.
//   scan   the 16 waves walk the (head, 16-column) tiles; per lane group of 16 lanes, 4 columns
//          stream through registers as in gdn_scan.hip's single-token path (state loads in flight,
//          each column reduced, updated and written back in turn).  A wave's first tile is loaded
//          before the conv phase, each further tile before the previous one is computed.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

struct DecodeArgs {
    const void* x;
    const void* cw;
    const void* cbias;
    const void* cst_in;  // not restrict: may alias cst_out
    void* cst_out;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    const float* state_in;  // not restrict: may alias state_out
    void* out;
    float* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    int B, N, HQ, H, K, V, C, G, W, D, L;
    int gate_dtype;
    uint32_t flags;
    int silu;
    float scale;
    int n_blocks;
};

constexpr int kMaxL = 4;  // (W-1)*D handled by this kernel

// Waves per block (one (sequence, key head) per block).
#ifndef GDN_DECODE_STEP_NW
#define GDN_DECODE_STEP_NW 4
#endif
// Grids with fewer blocks than compute units run 8 waves per block instead.
constexpr long long kSmallGridBlocks = 256;

// Whole-call checks: the offsets (as everywhere) and, for this entry point, at most one token per
// sequence.  Returns 0, GDN_ERR_OFFSETS or GDN_ERR_UNSUPPORTED; must be reached by all threads.
__device__ __forceinline__ int decode_call_status(const int32_t* __restrict__ offsets, int B, int N) {
    int bad = 0, long_seq = 0;
    for (int i = threadIdx.x; i <= B; i += blockDim.x) {
        const int o = offsets[i];
        if (i == 0) bad |= (o != 0);
        else {
            const int prev = offsets[i - 1];
            bad |= (prev > o);
            long_seq |= (o - prev > 1);
        }
        if (i == B) bad |= (o != N);
    }
    if (__syncthreads_or(bad)) return GDN_ERR_OFFSETS;
    if (__syncthreads_or(long_seq)) return GDN_ERR_UNSUPPORTED;
    return 0;
}

template <typename T, typename S, int K, int LPC, int CPL, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(DecodeArgs p) {
    constexpr int EPL = K / LPC;
    static_assert(EPL % 4 == 0, "whole 16-byte chunks per lane");
    constexpr int GPW = 64 / LPC;
    constexpr int WC = GPW * CPL;  // columns per wave tile
    constexpr int NT = 64 * NW;
    using TS = typename T::storage;
    using SS = typename S::storage;
    extern __shared__ float ylds[];  // [q: K | k: K | v: G*V], the conv outputs of this block
    float* const yq = ylds;
    float* const yk = ylds + K;
    float* const yv = ylds + 2 * K;

    const int status = decode_call_status(p.offsets, p.B, p.N);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.dev_status != nullptr) *p.dev_status = status ? status : GDN_OK;
    if (status) return;

    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, 1);
    const int kh = blk % p.HQ;
    const int b = blk / p.HQ;
    const int GV = p.G * p.V;  // value columns of this block
    const int start = p.offsets[b];
    const int len = p.offsets[b + 1] - start;  // 0 or 1
    const int tid = (int)threadIdx.x;

    // the first state tile of each wave does not depend on the conv: its loads go out first and are
    // in flight during the conv phase
    const int wave = tid / 64, lane = tid % 64;
    const int grp = lane / LPC, gl = lane % LPC;
    const int n_tiles = (GV + WC - 1) / WC;
    const bool has_state = p.state_in != nullptr;
    // state columns of tile tl for this lane group: global column gc = tl*WC + grp*CPL + c of the
    // block's G*V columns -> head kh*G + gc/V, column gc%V (a group never straddles heads: V % CPL == 0)
    auto col_ptr = [&](int gc) { return ((size_t)b * p.H + (size_t)kh * p.G) * p.V + gc; };
    auto load_tile = [&](int tl, f32x4 (&dst)[CPL][EPL / 4]) {
        const int gc0 = min(tl * WC + grp * CPL, GV - CPL);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float* sp = p.state_in + col_ptr(gc0 + c) * K;
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i) dst[c][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + 4 * (gl + LPC * i)));
        }
    };
    f32x4 ta[CPL][EPL / 4], tb[CPL][EPL / 4];
    if (wave < n_tiles && has_state) load_tile(wave, ta);

    // ---- conv ------------------------------------------------------------------------------------------
    // The block's NCH = 2K + G*V channels are three contiguous channel ranges (q of kh, k of kh, v of
    // heads kh*G ..), so their windows, weights, token values and biases are contiguous too: all
    // threads copy them into LDS with consecutive lanes on consecutive elements, then one thread per
    // channel computes the output and the new window is written back the same way.
    const int NCH = 2 * K + GV;
    const int L = p.L, W = p.W, D = p.D;
    const int seg_g[3] = {kh * K, p.HQ * K + kh * K, 2 * p.HQ * K + kh * GV};  // first global channel
    const int seg_l[3] = {0, K, 2 * K};                                      // first block channel
    const int seg_n[3] = {K, K, GV};
    SS* const lwin = reinterpret_cast<SS*>(ylds + NCH);                     // [NCH][L]
    TS* const lw = reinterpret_cast<TS*>(lwin + ((NCH * L + 1) & ~1));     // [NCH][W]
    TS* const lx = lw + ((NCH * W + 1) & ~1);                               // [NCH]
    TS* const lb = lx + NCH;                                                // [NCH]
    const SS* wi = static_cast<const SS*>(p.cst_in);
    const TS* const xg = static_cast<const TS*>(p.x);
    const TS* const wg = static_cast<const TS*>(p.cw);
    const TS* const bg = static_cast<const TS*>(p.cbias);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        const size_t wsrc = ((size_t)b * p.C + seg_g[g]) * L;
        for (int e = tid; e < seg_n[g] * L; e += NT) lwin[seg_l[g] * L + e] = wi != nullptr ? wi[wsrc + e] : SS();
        if (len == 1) {
            for (int e = tid; e < seg_n[g] * W; e += NT) lw[seg_l[g] * W + e] = wg[(size_t)seg_g[g] * W + e];
            for (int e = tid; e < seg_n[g]; e += NT) {
                lx[seg_l[g] + e] = xg[(size_t)start * p.C + seg_g[g] + e];
                lb[seg_l[g] + e] = bg != nullptr ? bg[seg_g[g] + e] : TS();
            }
        }
    }
    __syncthreads();
    if (len == 1) {
        for (int c = tid; c < NCH; c += NT) {
            float acc = bg != nullptr ? to_f32<T>(lb[c]) : 0.0f;
            for (int j = 0; j < W; ++j) {
                // tap j of the sequence's first token reads window entry j*D, tap W-1 the token
                const float xv = j == W - 1 ? to_f32<T>(lx[c]) : to_f32<S>(lwin[c * L + j * D]);
                acc = fmaf(to_f32<T>(lw[c * W + j]), xv, acc);
            }
            if (p.silu) acc = acc * __builtin_amdgcn_rcpf(1.0f + __expf(-acc));
            ylds[c] = to_f32<T>(from_f32<T>(acc));  // the conv output as the 2-call chain stores it
        }
    }
    if (p.cst_out != nullptr && L > 0) {
        // new window entry j = (old window ++ the 0 or 1 tokens)[j + len]; the old window is all in LDS,
        // so an aliased (in-place) window is updated correctly
        SS* const wo = static_cast<SS*>(p.cst_out);
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            const size_t wdst = ((size_t)b * p.C + seg_g[g]) * L;
            for (int e = tid; e < seg_n[g] * L; e += NT) {
                const int cl = e / L, j = e - cl * L;
                const int c = seg_l[g] + cl;
                SS v;
                if (j + len < L) {
                    v = lwin[c * L + j + len];
                } else if constexpr (std::is_same<S, T>::value) {
                    v = lx[c];
                } else {
                    v = to_f32<T>(lx[c]);  // exact widening into an fp32 window
                }
                wo[wdst + e] = v;
            }
        }
    }
    __syncthreads();

    // ---- recurrence over the block's (head, column) tiles ------------------------------------------

    float q[EPL], k[EPL];
    float rq = 1.0f, rk = 1.0f, qk = 0.0f;
    if (len == 1) {
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                q[4 * i + e] = yq[4 * (gl + LPC * i) + e];
                k[4 * i + e] = yk[4 * (gl + LPC * i) + e];
            }
        float nq = 0.0f, nk = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qk = fmaf(q[e], k[e], qk);
            nq = fmaf(q[e], q[e], nq);
            nk = fmaf(k[e], k[e], nk);
        }
        qk = group_sum<LPC>(qk);
        if (p.flags & GDN_L2NORM) {
            rq = rsqrtf(group_sum<LPC>(nq) + 1e-12f);
            rk = rsqrtf(group_sum<LPC>(nk) + 1e-12f);
        }
    }
    const float oscale = p.scale * rq;
    const bool softplus = (p.flags & GDN_SOFTPLUS) != 0;
    const float rmul = (p.flags & GDN_NO_RETRIEVE) ? 0.0f : 1.0f;  // the retrieval term's weight

    auto run_tile = [&](int tl, const f32x4 (&st)[CPL][EPL / 4]) {
        const int gc0 = tl * WC + grp * CPL;
        if (gc0 >= GV) return;
        const int hh = kh * p.G + gc0 / p.V;
        const int v0 = gc0 % p.V;
        float* const so = p.state_out;
        if (len == 0) {
            if (so == nullptr) return;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float* sp = so + col_ptr(gc0 + c) * K;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i)
                    __builtin_nontemporal_store(p.state_in ? st[c][i] : f32x4{0.f, 0.f, 0.f, 0.f},
                                                reinterpret_cast<f32x4*>(sp + 4 * (gl + LPC * i)));
            }
            return;
        }
        const size_t gi = (size_t)start * p.H + hh;
        float g = 1.0f;
        if (p.a) {
            const float ga = load_any(p.a, p.gate_dtype, gi);
            g = softplus ? expf(-expf(p.A_log[hh]) * softplus_f(ga + p.dt_bias[hh])) : expf(ga);
        }
        float beta = 1.0f;
        if (p.b) {
            const float gb = load_any(p.b, p.gate_dtype, gi);
            beta = (p.flags & GDN_SIGMOID) ? 1.0f / (1.0f + expf(-gb)) : gb;
        }
        float mine = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float s[EPL];
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * i + e] = p.state_in ? st[c][i][e] : 0.0f;
            float pk = 0.0f, pq = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                pk = fmaf(s[e], k[e], pk);
                pq = fmaf(s[e], q[e], pq);
            }
            pk = group_sum<LPC>(pk);
            pq = group_sum<LPC>(pq);
            const float r = rmul * (g * rk * pk);
            const float dk = beta * (yv[gc0 + c] - r) * rk;
            const float o = oscale * fmaf(g, pq, dk * qk);
            if (so != nullptr) {
                float* sp = so + col_ptr(gc0 + c) * K;
#pragma unroll
                for (int i = 0; i < EPL / 4; ++i) {
                    f32x4 nv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) nv[e] = fmaf(dk, k[4 * i + e], g * s[4 * i + e]);
                    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(sp + 4 * (gl + LPC * i)));
                }
            }
            if (gl == c) mine = o;
        }
        if (gl < CPL) static_cast<TS*>(p.out)[((size_t)start * p.H + hh) * p.V + v0 + gl] = from_f32<T>(mine);
    };

    // tiles wave, wave + NW, ...: the next tile's loads are issued before the current one is computed
    int tl = wave;
    while (tl < n_tiles) {
        if (tl + NW < n_tiles && has_state) load_tile(tl + NW, tb);
        run_tile(tl, ta);
        tl += NW;
        if (tl >= n_tiles) break;
        if (tl + NW < n_tiles && has_state) load_tile(tl + NW, ta);
        run_tile(tl, tb);
        tl += NW;
    }
}

// LDS of one block: conv outputs (fp32), then the staged windows, weights, token values and biases.
inline size_t decode_lds_bytes(int K, int GV, int L, int W, size_t s_window) {
    const size_t nch = 2 * (size_t)K + GV;
    return nch * 4 + ((nch * L + 1) & ~(size_t)1) * s_window + ((nch * W + 1) & ~(size_t)1) * 4 + 2 * nch * 4;
}

template <typename T, typename S, int K>
hipError_t launch_k(DecodeArgs p, hipStream_t stream) {
    constexpr int LPC = K >= 64 ? 16 : 8;
    constexpr int CPL = K >= 256 ? 2 : 4;
    constexpr int NW = GDN_DECODE_STEP_NW;
    const long long blocks = (long long)p.B * p.HQ;
    if (blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    p.n_blocks = (int)blocks;
    const size_t lds = decode_lds_bytes(K, p.G * p.V, p.L, p.W, sizeof(typename S::storage));
    // A grid smaller than the chip (small batches, where this single launch is the faster form)
    // gives each block 8 waves, so twice the column tiles of a block are in flight at once
    // (B = 8: 25.3 -> 21.6 us per step; 16 waves spill and gain nothing more).
    if (blocks < kSmallGridBlocks)
        hipLaunchKernelGGL((decode_kernel<T, S, K, LPC, CPL, 8>), dim3((unsigned)blocks), dim3(64 * 8), lds, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<T, S, K, LPC, CPL, NW>), dim3((unsigned)blocks), dim3(64 * NW), lds, stream, p);
    return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_ts(const DecodeArgs& p, hipStream_t stream) {
    switch (p.K) {
        case 32: return launch_k<T, S, 32>(p, stream);
        case 64: return launch_k<T, S, 64>(p, stream);
        case 128: return launch_k<T, S, 128>(p, stream);
        case 256: return launch_k<T, S, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_step_supported(int K, int V, int G, int W, int D) {
    // a block stages its channels' conv inputs and outputs in LDS: at most 64 KB (worst case of the
    // element sizes counted)
    if (!(K == 32 || K == 64 || K == 128 || K == 256) || V % 4 != 0 || (long long)(W - 1) * D > kMaxL) return false;
    if ((long long)G * V > (1 << 20)) return false;
    return decode_lds_bytes(K, G * V, (W - 1) * D, W, 4) <= 65536;
}

hipError_t launch_decode_step(const DecodeStepLaunch& a, hipStream_t stream) {
    DecodeArgs p;
    p.x = a.x;
    p.cw = a.conv_w;
    p.cbias = a.conv_bias;
    p.cst_in = a.conv_state_in;
    p.cst_out = a.conv_state_out;
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
    p.C = 2 * a.HQ * a.K + a.H * a.V;
    p.G = a.H / a.HQ;
    p.W = a.W;
    p.D = a.D;
    p.L = (a.W - 1) * a.D;
    p.gate_dtype = a.gate_dtype;
    p.flags = a.flags;
    p.silu = a.silu ? 1 : 0;
    p.scale = a.scale;
    p.n_blocks = 0;
    const bool wide = a.state_dtype == GDN_F32;
    switch (a.qkv_dtype) {
        case GDN_F32: return launch_ts<F32, F32>(p, stream);
        case GDN_BF16: return wide ? launch_ts<BF16, F32>(p, stream) : launch_ts<BF16, BF16>(p, stream);
        case GDN_F16: return wide ? launch_ts<F16, F32>(p, stream) : launch_ts<F16, F16>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
