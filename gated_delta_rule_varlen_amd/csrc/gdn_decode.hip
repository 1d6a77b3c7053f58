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
// Two forms.
// Key-head form (small batches, and any call that updates the window in place): a block owns
// (sequence b, key head kh): the q/k channels of kh and every value column of the G value heads
// that read kh, so that each carried window entry has exactly one reader and one writer (the q/k
// windows are shared by the G heads; with an in-place window, a split over blocks would race).
//   conv   the block's channels (q and k of kh, v of its heads) are staged in LDS with 16-byte
//          accesses where aligned, one thread computes each output, rounded to the I/O type, and
//          the new window is written back the same way.
//   scan   the waves walk the (head, 16-column) tiles; per lane group of 16 lanes, 4 columns
//          stream through registers as in gdn_scan.hip's single-token path (state loads in flight,
//          each column reduced, updated and written back in turn).  A wave's first tile is loaded
//          before the conv phase, each further tile before the previous one is computed.
// Column-tile form (large batches with a separate new window): a block owns (sequence, value
// head, 128 columns), one 16-column tile per wave; it recomputes its key head's q/k conv outputs
// (identical in every block) and its columns' v outputs.  The conv inputs are loaded into
// registers first, then the state columns, so the conv waits only for its own inputs.
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
    int n_vtiles;  // column-tile form: column tiles per (sequence, value head)
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

// Cooperative copy of n elements from global memory to LDS: 16 bytes per thread access when both
// ends are 16-byte aligned and the size is whole 16-byte units (block-uniform), element-wise
// otherwise.
template <typename E>
__device__ __forceinline__ void stage_copy(E* lds, const E* g, int n, int tid, int nt) {
    const bool vec = (((uintptr_t)g | (uintptr_t)lds) & 15) == 0 && (n * (int)sizeof(E)) % 16 == 0;
    if (vec) {
        const int nv = n * (int)sizeof(E) / 16;
        for (int i = tid; i < nv; i += nt) reinterpret_cast<u32x4*>(lds)[i] = reinterpret_cast<const u32x4*>(g)[i];
    } else {
        for (int i = tid; i < n; i += nt) lds[i] = g[i];
    }
}
// 16-byte-aligned element offset in LDS after `bytes` bytes
__host__ __device__ constexpr size_t lds_align16(size_t bytes) { return (bytes + 15) & ~(size_t)15; }

#ifndef GDN_DECODE_STEP_MINW
#define GDN_DECODE_STEP_MINW 4
#endif
// NW = 4: GDN_DECODE_STEP_MINW blocks per compute unit, so a block's conv phase hides behind the
// others' state streams.
template <typename T, typename S, int K, int LPC, int CPL, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? GDN_DECODE_STEP_MINW : 1) void decode_kernel(DecodeArgs p) {
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
    // regions start 16-byte aligned (the segments inside them too: K is a multiple of 32)
    char* const lbase = reinterpret_cast<char*>(ylds);
    SS* const lwin = reinterpret_cast<SS*>(lbase + lds_align16((size_t)NCH * 4));        // [NCH][L]
    TS* const lw = reinterpret_cast<TS*>(reinterpret_cast<char*>(lwin) + lds_align16((size_t)NCH * L * sizeof(SS)));
    TS* const lx = reinterpret_cast<TS*>(reinterpret_cast<char*>(lw) + lds_align16((size_t)NCH * W * sizeof(TS)));
    TS* const lb = reinterpret_cast<TS*>(reinterpret_cast<char*>(lx) + lds_align16((size_t)NCH * sizeof(TS)));
    const SS* wi = static_cast<const SS*>(p.cst_in);
    const TS* const xg = static_cast<const TS*>(p.x);
    const TS* const wg = static_cast<const TS*>(p.cw);
    const TS* const bg = static_cast<const TS*>(p.cbias);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        if (wi != nullptr) stage_copy(lwin + seg_l[g] * L, wi + ((size_t)b * p.C + seg_g[g]) * L, seg_n[g] * L, tid, NT);
        else
            for (int e = tid; e < seg_n[g] * L; e += NT) lwin[seg_l[g] * L + e] = SS();
        if (len == 1) {
            stage_copy(lw + seg_l[g] * W, wg + (size_t)seg_g[g] * W, seg_n[g] * W, tid, NT);
            stage_copy(lx + seg_l[g], xg + (size_t)start * p.C + seg_g[g], seg_n[g], tid, NT);
            if (bg != nullptr) stage_copy(lb + seg_l[g], bg + seg_g[g], seg_n[g], tid, NT);
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
        // so an aliased (in-place) window is updated correctly.  Written 16 bytes per thread access
        // when the segment allows it.
        SS* const wo = static_cast<SS*>(p.cst_out);
        auto entry = [&](int g, int e) {
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
            return v;
        };
        constexpr int EV = 16 / (int)sizeof(SS);  // window entries per 16 bytes
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            SS* const dst = wo + ((size_t)b * p.C + seg_g[g]) * L;
            const int n = seg_n[g] * L;
            if ((((uintptr_t)dst) & 15) == 0 && n % EV == 0) {
                for (int v = tid; v < n / EV; v += NT) {
                    union {
                        u32x4 u;
                        SS e[EV];
                    } pk;
#pragma unroll
                    for (int i = 0; i < EV; ++i) pk.e[i] = entry(g, EV * v + i);
                    reinterpret_cast<u32x4*>(dst)[v] = pk.u;
                }
            } else {
                for (int e = tid; e < n; e += NT) dst[e] = entry(g, e);
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

// Column-tile form: a block owns (sequence b, value head h, BC value columns), as the DECODE
// kernel's blocks do, so that a large batch streams its state through many short-lived blocks.  Each
// block recomputes the q/k conv outputs of its key head (2K channels, the same arithmetic, so the
// same values in every block) and the conv outputs of its own value columns; the q/k window is
// written back by the head group's first block (h % G == 0, first column tile) and each value
// window by the block of its columns, so every window entry still has one writer.
template <typename T, typename S, int K, int LPC, int CPL, int NW>
#ifndef GDN_DECODE_COL_MINW
#define GDN_DECODE_COL_MINW 4
#endif
__global__ __launch_bounds__(64 * NW, GDN_DECODE_COL_MINW) void decode_col_kernel(DecodeArgs p) {
    constexpr int EPL = K / LPC;
    static_assert(EPL % 4 == 0, "whole 16-byte chunks per lane");
    constexpr int GPW = 64 / LPC;
    constexpr int WC = GPW * CPL;  // columns per wave
    constexpr int BC = NW * WC;    // columns per block
    constexpr int NT = 64 * NW;
    using TS = typename T::storage;
    using SS = typename S::storage;
    extern __shared__ float ylds[];  // [q: K | k: K | v: BC], the conv outputs of this block
    float* const yq = ylds;
    float* const yk = ylds + K;
    float* const yv = ylds + 2 * K;

    const int status = decode_call_status(p.offsets, p.B, p.N);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.dev_status != nullptr) *p.dev_status = status ? status : GDN_OK;
    if (status) return;

    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, p.G * p.n_vtiles);
    const int vt = blk % p.n_vtiles;
    const int bh = blk / p.n_vtiles;
    const int h = bh % p.H;
    const int b = bh / p.H;
    const int kh = h / p.G;
    const int start = p.offsets[b];
    const int len = p.offsets[b + 1] - start;  // 0 or 1
    const int tid = (int)threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int grp = lane / LPC, gl = lane % LPC;
    const int cbase = vt * BC;                     // first value column of the block
    const int nvb = min(BC, p.V - cbase);          // value columns of the block
    const int v0 = cbase + wave * WC + grp * CPL;  // first column of this lane group
    const size_t col0 = ((size_t)b * p.H + h) * p.V;

    f32x4 st[CPL][EPL / 4];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) st[c][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the state columns do not depend on the conv: their loads are issued right after the conv
    // inputs', so waiting for the conv inputs never waits for the state
    auto load_state = [&]() {
        if (p.state_in == nullptr) return;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (v0 + c >= p.V) continue;
            const float* sp = p.state_in + (col0 + v0 + c) * K;
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i)
                st[c][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + 4 * (gl + LPC * i)));
        }
    };

    // ---- conv of the block's channels: q and k of kh, v of its columns -------------------------------
    const int NCH = 2 * K + nvb;
    const int L = p.L, W = p.W, D = p.D;
    const int seg_g[3] = {kh * K, p.HQ * K + kh * K, 2 * p.HQ * K + h * p.V + cbase};  // first global channel
    const int seg_l[3] = {0, K, 2 * K};                                               // first block channel
    const int seg_n[3] = {K, K, nvb};
    const bool own_qk = (h % p.G) == 0 && vt == 0;  // this block writes the q/k window back
    char* const lbase = reinterpret_cast<char*>(ylds);
    const int NCHM = 2 * K + BC;  // region sizes use the block's maximum channel count
    SS* const lwin = reinterpret_cast<SS*>(lbase + lds_align16((size_t)NCHM * 4));  // [NCH][L]
    TS* const lw = reinterpret_cast<TS*>(reinterpret_cast<char*>(lwin) + lds_align16((size_t)NCHM * L * sizeof(SS)));
    TS* const lx = reinterpret_cast<TS*>(reinterpret_cast<char*>(lw) + lds_align16((size_t)NCHM * W * sizeof(TS)));
    TS* const lb = reinterpret_cast<TS*>(reinterpret_cast<char*>(lx) + lds_align16((size_t)NCHM * sizeof(TS)));
    const SS* wi = static_cast<const SS*>(p.cst_in);
    const TS* const xg = static_cast<const TS*>(p.x);
    const TS* const wg = static_cast<const TS*>(p.cw);
    const TS* const bg = static_cast<const TS*>(p.cbias);
    // The conv inputs are up to 12 contiguous ranges (window, weights, token, bias of each segment).
    // When every range is whole, 16-byte aligned units they go through registers, 16 bytes a thread
    // access, with the state loads issued between the loads and the LDS writes; otherwise element by
    // element after the state loads.
    // range 4g + {0, 1, 2, 3}: window, weights, token, bias of segment g (0 units when absent); the
    // ranges sit at fixed indices so that every index below is a compile-time constant
    constexpr int MAXR = 12;
    const char* rsrc[MAXR];
    char* rdst[MAXR];
    int rn[MAXR];  // 16-byte units
    bool vec = true;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        const void* src[4] = {wi ? (const void*)(wi + ((size_t)b * p.C + seg_g[g]) * L) : nullptr,
                              (const void*)(wg + (size_t)seg_g[g] * W),
                              (const void*)(xg + (size_t)start * p.C + seg_g[g]),
                              bg ? (const void*)(bg + seg_g[g]) : nullptr};
        void* dst[4] = {lwin + seg_l[g] * L, lw + seg_l[g] * W, lx + seg_l[g], lb + seg_l[g]};
        const int bytes[4] = {wi ? seg_n[g] * L * (int)sizeof(SS) : 0, len == 1 ? seg_n[g] * W * (int)sizeof(TS) : 0,
                              len == 1 ? seg_n[g] * (int)sizeof(TS) : 0,
                              (len == 1 && bg) ? seg_n[g] * (int)sizeof(TS) : 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            rsrc[r] = static_cast<const char*>(src[i]);
            rdst[r] = static_cast<char*>(dst[i]);
            rn[r] = bytes[i] / 16;
            if (bytes[i] > 0) vec = vec && ((((uintptr_t)src[i]) | ((uintptr_t)dst[i])) & 15) == 0 && bytes[i] % 16 == 0;
        }
    }
    // units per thread: (2K + BC) channels x (4 window entries + 5 weights + token + bias) x 4 bytes
    constexpr int MAXU = ((2 * K + BC) * 44 / 16 + NT - 1) / NT;
    int total = 0;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) total += rn[r];
    vec = vec && total <= MAXU * NT;
    if (vec) {
        u32x4 reg[MAXU];
        // source and destination of unit u: a walk over the fixed ranges
        auto unit = [&](int u, const u32x4*& src, u32x4*& dst) {
            int off = u;
            bool found = false;
#pragma unroll
            for (int r = 0; r < MAXR; ++r) {
                if (!found) {
                    if (off < rn[r]) {
                        src = reinterpret_cast<const u32x4*>(rsrc[r]) + off;
                        dst = reinterpret_cast<u32x4*>(rdst[r]) + off;
                        found = true;
                    } else {
                        off -= rn[r];
                    }
                }
            }
        };
#pragma unroll
        for (int j = 0; j < MAXU; ++j) {
            const int u = tid + j * NT;
            if (u < total) {
                const u32x4* src = nullptr;
                u32x4* dst = nullptr;
                unit(u, src, dst);
                reg[j] = *src;
            }
        }
        load_state();
#pragma unroll
        for (int j = 0; j < MAXU; ++j) {
            const int u = tid + j * NT;
            if (u < total) {
                const u32x4* src = nullptr;
                u32x4* dst = nullptr;
                unit(u, src, dst);
                *dst = reg[j];
            }
        }
    } else {
        load_state();
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            if (len == 1) {
                stage_copy(lw + seg_l[g] * W, wg + (size_t)seg_g[g] * W, seg_n[g] * W, tid, NT);
                stage_copy(lx + seg_l[g], xg + (size_t)start * p.C + seg_g[g], seg_n[g], tid, NT);
                if (bg != nullptr) stage_copy(lb + seg_l[g], bg + seg_g[g], seg_n[g], tid, NT);
            }
            if (wi != nullptr) stage_copy(lwin + seg_l[g] * L, wi + ((size_t)b * p.C + seg_g[g]) * L, seg_n[g] * L, tid, NT);
        }
    }
    if (wi == nullptr)
        for (int e = tid; e < NCH * L; e += NT) lwin[e] = SS();
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
        // new window entry j = (old window ++ the 0 or 1 tokens)[j + len], from the old window in LDS
        SS* const wo = static_cast<SS*>(p.cst_out);
        auto entry = [&](int g, int e) {
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
            return v;
        };
        constexpr int EV = 16 / (int)sizeof(SS);  // window entries per 16 bytes
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            if (g < 2 && !own_qk) continue;
            SS* const dst = wo + ((size_t)b * p.C + seg_g[g]) * L;
            const int n = seg_n[g] * L;
            if ((((uintptr_t)dst) & 15) == 0 && n % EV == 0) {
                for (int v = tid; v < n / EV; v += NT) {
                    union {
                        u32x4 u;
                        SS e[EV];
                    } pk;
#pragma unroll
                    for (int i = 0; i < EV; ++i) pk.e[i] = entry(g, EV * v + i);
                    reinterpret_cast<u32x4*>(dst)[v] = pk.u;
                }
            } else {
                for (int e = tid; e < n; e += NT) dst[e] = entry(g, e);
            }
        }
    }
    __syncthreads();

    // ---- the recurrence of the lane group's columns --------------------------------------------------
    float* const so = p.state_out;
    if (len == 0) {
        if (so == nullptr) return;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (v0 + c >= p.V) continue;
            float* sp = so + (col0 + v0 + c) * K;
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i)
                __builtin_nontemporal_store(st[c][i], reinterpret_cast<f32x4*>(sp + 4 * (gl + LPC * i)));
        }
        return;
    }
    float q[EPL], k[EPL];
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q[4 * i + e] = yq[4 * (gl + LPC * i) + e];
            k[4 * i + e] = yk[4 * (gl + LPC * i) + e];
        }
    float qk = 0.0f, nq = 0.0f, nk = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        qk = fmaf(q[e], k[e], qk);
        nq = fmaf(q[e], q[e], nq);
        nk = fmaf(k[e], k[e], nk);
    }
    qk = group_sum<LPC>(qk);
    float rq = 1.0f, rk = 1.0f;
    if (p.flags & GDN_L2NORM) {
        rq = rsqrtf(group_sum<LPC>(nq) + 1e-12f);
        rk = rsqrtf(group_sum<LPC>(nk) + 1e-12f);
    }
    const float oscale = p.scale * rq;
    const float rmul = (p.flags & GDN_NO_RETRIEVE) ? 0.0f : 1.0f;  // the retrieval term's weight
    const size_t gi = (size_t)start * p.H + h;
    float g = 1.0f;
    if (p.a) {
        const float ga = load_any(p.a, p.gate_dtype, gi);
        g = (p.flags & GDN_SOFTPLUS) ? expf(-expf(p.A_log[h]) * softplus_f(ga + p.dt_bias[h])) : expf(ga);
    }
    float beta = 1.0f;
    if (p.b) {
        const float gb = load_any(p.b, p.gate_dtype, gi);
        beta = (p.flags & GDN_SIGMOID) ? 1.0f / (1.0f + expf(-gb)) : gb;
    }
    float mine = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (v0 + c >= p.V) continue;
        float s[EPL];
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * i + e] = st[c][i][e];
        float pk = 0.0f, pq = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            pk = fmaf(s[e], k[e], pk);
            pq = fmaf(s[e], q[e], pq);
        }
        pk = group_sum<LPC>(pk);
        pq = group_sum<LPC>(pq);
        const float r = rmul * (g * rk * pk);
        const float dk = beta * (yv[v0 - cbase + c] - r) * rk;
        const float o = oscale * fmaf(g, pq, dk * qk);
        if (so != nullptr) {
            float* sp = so + (col0 + v0 + c) * K;
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
    if (gl < CPL && v0 + gl < p.V) static_cast<TS*>(p.out)[gi * p.V + v0 + gl] = from_f32<T>(mine);
}

// LDS of one block: conv outputs (fp32), then the staged windows, weights, token values and biases,
// each region 16-byte aligned (element sizes counted at 4 bytes for the I/O type: the worst case).
inline size_t decode_lds_bytes(int K, int GV, int L, int W, size_t s_window) {
    const size_t nch = 2 * (size_t)K + GV;
    return lds_align16(nch * 4) + lds_align16(nch * L * s_window) + lds_align16(nch * W * 4) + 2 * lds_align16(nch * 4);
}

template <typename T, typename S, int K>
hipError_t launch_k(DecodeArgs p, hipStream_t stream) {
    constexpr int LPC = K >= 64 ? 16 : 8;
    constexpr int CPL = K >= 256 ? 2 : 4;
    constexpr int NW = GDN_DECODE_STEP_NW;
    const long long blocks = (long long)p.B * p.HQ;
    if (blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    p.n_blocks = (int)blocks;
    // Large batches with a separate new window: the column-tile form (many short-lived blocks
    // stream the state; several blocks read a key head's q/k window, so the window may not be
    // updated in place).  Measured at B = 256, H = 32, K = V = 128, bf16: 185 us per step against
    // 224 us for the key-head form and 191 us for the two-launch chain.
    const size_t wbytes = (size_t)p.B * p.C * p.L * sizeof(typename S::storage);
    const char* wi = static_cast<const char*>(p.cst_in);
    const char* wo = static_cast<const char*>(p.cst_out);
    const bool window_aliased = wi != nullptr && wo != nullptr && p.L > 0 && wi < wo + wbytes && wo < wi + wbytes;
    if (blocks >= kSmallGridBlocks && !window_aliased) {
#ifndef GDN_DECODE_COL_NW
#define GDN_DECODE_COL_NW 8
#endif
        constexpr int CNW = GDN_DECODE_COL_NW;
        constexpr int BC = CNW * (64 / LPC) * CPL;
        p.n_vtiles = (p.V + BC - 1) / BC;
        const long long cblocks = (long long)p.B * p.H * p.n_vtiles;
        if (cblocks > kMaxBlocks) return hipErrorInvalidConfiguration;
        p.n_blocks = (int)cblocks;
        const size_t clds = decode_lds_bytes(K, BC, p.L, p.W, sizeof(typename S::storage));
        hipLaunchKernelGGL((decode_col_kernel<T, S, K, LPC, CPL, CNW>), dim3((unsigned)cblocks), dim3(64 * CNW), clds, stream,
                           p);
        return hipGetLastError();
    }
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
    p.n_vtiles = 0;
    const bool wide = a.state_dtype == GDN_F32;
    switch (a.qkv_dtype) {
        case GDN_F32: return launch_ts<F32, F32>(p, stream);
        case GDN_BF16: return wide ? launch_ts<BF16, F32>(p, stream) : launch_ts<BF16, BF16>(p, stream);
        case GDN_F16: return wide ? launch_ts<F16, F32>(p, stream) : launch_ts<F16, F16>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
