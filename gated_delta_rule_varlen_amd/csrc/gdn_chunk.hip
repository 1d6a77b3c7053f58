// gdn_chunk.hip -- chunked (WY / UT-transform) form of the gated delta-rule recurrence (gfx950).
//
// Operation: paged_ssm.rs page, kernel string DELTA, which the host fn delta() runs chunked for long
// prefills.  The chunked kernel's source is not on the pages, so the algebra below is derived from
// the recurrence itself.  In matrix form (S is V x K, row v = the state of value column v)
//     S_t = g_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,     o_t = scale S_t q_t.
// For one chunk of C = 64 tokens of one sequence and head, with G_i the cumulative log-decay inside
// the chunk and S0 the state entering it:
//     A_ij = b_i e^{G_i - G_j} (k_i . k_j)  (j < i),   T = (I + A)^{-1}   (unit lower triangular)
//     W  = T diag(b e^G) K,      U' = T diag(b) V,      U = U' - W S0^T   (U row i = delta_i)
//     O  = scale [ diag(e^G) Q S0^T + (M o Q K^T) U ],  M_ij = e^{G_i - G_j} (j <= i), else 0
//     S_C = e^{G_C} S0 + U^T diag(e^{G_C - G}) K.
// Only decays that are finite and positive are allowed (log-decays are summed), which the softplus
// gate guarantees.  Chunks never cross sequence boundaries.
//
// Kernels (all on the caller's stream; bf16 MFMA operands, fp32 accumulation, fp32 state):
//   index  one block: checks the offsets (nothing is written anywhere when they are malformed),
//          builds the table of each sequence's first chunk.
//   prep   one block per (chunk, head), parallel: gates, G, the normalised keys, A by MFMA
//          (K K^T), T by blocked inversion (16x16 diagonal blocks by substitution, off-diagonal
//          blocks by fp32 MFMA), W^T = X^T T^T and U' = T Y by MFMA.  Writes W, U'^T,
//          Kd^T = (diag(e^{G_C - G}) K)^T, G and the key norms to the workspace.
//   state  one block per (sequence, head, 16-column tile), sequential over the sequence's chunks:
//          U = U' - W S^T, S <- e^{G_C} S + U^T Kd.  The fp32 state stays in MFMA accumulators.
//          Writes U^T and the chunk-entry state S (bf16) to the workspace; the final state out.
//   out    one block per (chunk, head), parallel: O^T = diag-scaled S Q^T + U^T (M o Q K^T)^T.
//
// Every MFMA operand is staged "inner-dimension contiguous" so each lane's 8-element fragment is one
// 16-byte access (operand lane layouts of v_mfma_f32_16x16x32_bf16 / 16x16x4f32: lane l holds row
// l%16, inner elements 8*(l/16)..+7 (resp. l/16); accumulator lane l holds rows 4*(l/16)..+3 of
// column l%16).
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int CH = 64;  // tokens per chunk
// LDS rows holding MFMA fragments are padded by 16 bytes: a fragment read has the 16 lanes of a
// group on 16 consecutive rows, and unpadded 128- or 256-byte rows would put them all on the same
// four banks (a 16-way conflict); the pad shifts each row by four banks.
constexpr int PAD = 8;  // bf16 elements

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Scheduling hint for the current region: NR LDS reads first, then NM matrix products.  Issuing all
// reads of a phase up front lets their latencies overlap instead of stalling before every product.
template <int NR, int NM>
__device__ __forceinline__ void order_reads_then_mfma() {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// 16 rows x 32 inner elements starting at `base` (row stride ld elements): this lane's fragment.
__device__ __forceinline__ bf16x8 frag(const uint16_t* base, int ld, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + (lane & 15) * ld + 8 * (lane >> 4));
}
__device__ __forceinline__ uint16_t bf(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    return u32x2{(uint32_t)bf(a) | ((uint32_t)bf(b) << 16), (uint32_t)bf(c) | ((uint32_t)bf(d) << 16)};
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workspace layout (byte offsets), identical on host and device.
struct WsLayout {
    size_t hdr;      // int32: [0] status, [1] total chunks; cstart[B+1] at +64
    size_t w;        // W      [chunk-head][CH][K]  bf16
    size_t upt;      // U'^T   [chunk-head][V][CH]  bf16
    size_t kdt;      // Kd^T   [chunk-head][K][CH]  bf16, Kd = diag(e^{G_C - G}) Khat
    size_t pm;       // P      [chunk-head][CH][CH] bf16, P = M o (Qhat Khat^T)
    size_t gam;      // G      [chunk-head][CH]     f32
    size_t rq;       // 1/|q|  [chunk-head][CH]     f32
    size_t total;
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline WsLayout ws_layout(int B, int N, int H, int K, int V) {
    WsLayout L;
    const size_t nch = ((size_t)N + CH - 1) / CH + (size_t)B;  // upper bound on chunks over all sequences
    const size_t nh = nch * (size_t)H;
    size_t o = 0;
    L.hdr = o;
    o = align256(o + 64 + 4 * ((size_t)B + 1));
    L.w = o;
    o = align256(o + nh * CH * K * 2);
    L.upt = o;
    o = align256(o + nh * V * CH * 2);
    L.kdt = o;
    o = align256(o + nh * K * CH * 2);
    L.pm = o;
    o = align256(o + nh * CH * CH * 2);
    L.gam = o;
    o = align256(o + nh * CH * 4);
    L.rq = o;
    o = align256(o + nh * CH * 4);
    L.total = o;
    return L;
}

struct ChunkArgs {
    const void* qkv;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    const float* state_in;  // not restrict: may alias state_out
    void* out;
    float* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    char* ws;
    WsLayout L;
    int B, N, HQ, H, K, V, C, G;
    int gate_dtype;
    uint32_t flags;
    float scale;
    int n_blocks;
};

// ---- index: offsets check and the first-chunk table --------------------------------------------
__global__ __launch_bounds__(1024) void chunk_index_kernel(ChunkArgs p) {
    const bool malformed = offsets_malformed(p.offsets, p.B, p.N);
    report_status(p.dev_status, malformed);
    int32_t* hdr = reinterpret_cast<int32_t*>(p.ws + p.L.hdr);
    int32_t* cstart = hdr + 16;
    if (malformed) {
        if (threadIdx.x == 0) hdr[0] = GDN_ERR_OFFSETS;
        return;
    }
    __shared__ int warp_tot[16];
    __shared__ int carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int base = 0; base < p.B; base += 1024) {
        const int i = base + (int)threadIdx.x;
        const int cnt = i < p.B ? (p.offsets[i + 1] - p.offsets[i] + CH - 1) / CH : 0;
        int incl = cnt;  // inclusive scan inside the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) warp_tot[wv] = incl;
        __syncthreads();
        int before = carry;
        for (int k = 0; k < wv; ++k) before += warp_tot[k];
        if (i < p.B) cstart[i] = before + incl - cnt;
        __syncthreads();
        if (threadIdx.x == 1023) carry = before + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        cstart[p.B] = carry;
        hdr[1] = carry;
        hdr[0] = GDN_OK;
    }
}

// Sequence owning global chunk `cid` (the last b with cstart[b] <= cid); cid < total.
__device__ __forceinline__ int chunk_owner(const int32_t* cstart, int B, int cid) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cstart[mid] <= cid) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <typename T>
__device__ __forceinline__ void load8(const typename T::storage* p, float (&v)[8]) {
    if constexpr (std::is_same<T, F32>::value) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    } else {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = to_f32<T>((uint16_t)(raw[e] & 0xffffu));
            v[2 * e + 1] = to_f32<T>((uint16_t)(raw[e] >> 16));
        }
    }
}

__device__ __forceinline__ u32x4 pack8(const float* x, float s) {
    return u32x4{(uint32_t)bf(x[0] * s) | ((uint32_t)bf(x[1] * s) << 16), (uint32_t)bf(x[2] * s) | ((uint32_t)bf(x[3] * s) << 16),
                 (uint32_t)bf(x[4] * s) | ((uint32_t)bf(x[5] * s) << 16), (uint32_t)bf(x[6] * s) | ((uint32_t)bf(x[7] * s) << 16)};
}

// ---- prep ----------------------------------------------------------------------------------------
template <typename T, int K, int V>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ChunkArgs p) {
    using TS = typename T::storage;
    static_assert(K % 32 == 0 && V % 32 == 0 && K <= 128 && V <= 128, "chunk tile shapes");
    __shared__ __align__(16) uint16_t xt[K][CH + PAD];  // X^T = (diag(b e^G) Khat)^T
    __shared__ __align__(16) float am[CH][CH + 4];  // A (fp32); later T in bf16
    __shared__ __align__(16) union {
        struct {
            uint16_t kn[CH][K + PAD];  // Khat rows (bf16)
            uint16_t qn[CH][K + PAD];  // Qhat rows (bf16)
        } kq;                    // live until A and P are formed
        float tm[CH][CH + 4];    // T (fp32), until it is rounded to bf16
        uint16_t yt[V][CH + PAD];  // Y^T = (diag(b) V)^T, after that
    } u1;
    __shared__ __align__(16) float scr[4][16][17];
    __shared__ float s_gam[CH], s_beta[CH];
    uint16_t(*tb)[CH + PAD] = reinterpret_cast<uint16_t(*)[CH + PAD]>(&am[0][0]);  // T (bf16), once A is dead
    static_assert(sizeof(uint16_t) * CH * (CH + PAD) <= sizeof(float) * CH * (CH + 4), "T (bf16) fits in A's space");

    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.ws + p.L.hdr);
    if (hdr[0] != GDN_OK) return;
    const int total = hdr[1];
    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, p.G);
    const int cid = blk / p.H, h = blk % p.H;
    if (cid >= total) return;
    const int32_t* cstart = hdr + 16;
    const int b = chunk_owner(cstart, p.B, cid);
    const int t0 = p.offsets[b] + (cid - cstart[b]) * CH;
    const int n = min(CH, p.offsets[b + 1] - t0);
    const int kh = h / p.G;
    const size_t chh = (size_t)cid * p.H + h;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const TS* qkv = static_cast<const TS*>(p.qkv);

    // raw v rows, fetched now and staged once T is done (4 threads per token)
    constexpr int KPT = K / 4, VPT = V / 4;
    const int ti = tid >> 2, part = tid & 3;
    float vv[VPT];
#pragma unroll
    for (int e = 0; e < VPT; e += 8) {
        float t8[8];
        if (ti < n) load8<T>(qkv + (size_t)(t0 + ti) * p.C + (size_t)2 * p.HQ * K + (size_t)h * V + part * VPT + e, t8);
        else
#pragma unroll
            for (int z = 0; z < 8; ++z) t8[z] = 0.0f;
#pragma unroll
        for (int z = 0; z < 8; ++z) vv[e + z] = t8[z];
    }

    // gates and the cumulative log-decay (wave 0, one token per lane)
    if (wv == 0) {
        float ell = 0.0f, beta = 0.0f;
        if (lane < n) {
            const size_t gi = (size_t)(t0 + lane) * p.H + h;
            const float x = load_any(p.a, p.gate_dtype, gi);
            ell = -expf(p.A_log[h]) * softplus_f(x + p.dt_bias[h]);
            beta = 1.0f;
            if (p.b) {
                beta = load_any(p.b, p.gate_dtype, gi);
                if (p.flags & GDN_SIGMOID) beta = 1.0f / (1.0f + expf(-beta));
            }
        }
        float gam = ell;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(gam, d);
            if (lane >= d) gam += y;
        }
        s_gam[lane] = gam;
        s_beta[lane] = beta;
        reinterpret_cast<float*>(p.ws + p.L.gam)[chh * CH + lane] = gam;
    }
    // q and k rows: norms by a 4-lane reduction
    float kv[KPT], qv[KPT];
    float rq, rk;
    {
        float sk = 0.0f, sq = 0.0f;
#pragma unroll
        for (int e = 0; e < KPT; e += 8) {
            float tk[8], tq[8];
            if (ti < n) {
                const TS* row = qkv + (size_t)(t0 + ti) * p.C;
                load8<T>(row + (size_t)(p.HQ + kh) * K + part * KPT + e, tk);
                load8<T>(row + (size_t)kh * K + part * KPT + e, tq);
            } else {
#pragma unroll
                for (int z = 0; z < 8; ++z) tk[z] = tq[z] = 0.0f;
            }
#pragma unroll
            for (int z = 0; z < 8; ++z) {
                kv[e + z] = tk[z];
                qv[e + z] = tq[z];
                sk = fmaf(tk[z], tk[z], sk);
                sq = fmaf(tq[z], tq[z], sq);
            }
        }
        sk = group_sum<4>(sk);
        sq = group_sum<4>(sq);
        rk = rsqrtf(sk + 1e-12f);
        rq = rsqrtf(sq + 1e-12f);
        if (part == 0) reinterpret_cast<float*>(p.ws + p.L.rq)[chh * CH + ti] = rq;
    }
    __syncthreads();  // s_gam, s_beta ready
    {
        const float gi = s_gam[ti], gC = s_gam[CH - 1], bi = s_beta[ti];
        const float xs = bi * expf(gi), ks = expf(gC - gi);
        uint16_t* kdt = reinterpret_cast<uint16_t*>(p.ws + p.L.kdt) + chh * K * CH;
#pragma unroll
        for (int e = 0; e < KPT; e += 8) {
            *reinterpret_cast<u32x4*>(&u1.kq.kn[ti][part * KPT + e]) = pack8(&kv[e], rk);
            *reinterpret_cast<u32x4*>(&u1.kq.qn[ti][part * KPT + e]) = pack8(&qv[e], rq);
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int k = part * KPT + e;
            const float khat = kv[e] * rk;
            xt[k][ti] = bf(xs * khat);
            kdt[(size_t)k * CH + ti] = bf(ks * khat);
        }
    }
    __syncthreads();  // kn, qn, xt ready

    // Row block wv: A_ij = b_i e^{G_i - G_j} (khat_i . khat_j) for j < i, and
    // P_ij = e^{G_i - G_j} (qhat_i . khat_j) for j <= i (computed transposed: 4 consecutive j per lane)
    uint16_t* pout = reinterpret_cast<uint16_t*>(p.ws + p.L.pm) + chh * CH * CH;
    for (int jt = 0; jt < 4; ++jt) {
        f32x4 a = zero4(), pt = zero4();
        if (jt <= wv) {
#pragma unroll
            for (int kk = 0; kk < K; kk += 32) {
                const bf16x8 kj = frag(&u1.kq.kn[16 * jt][kk], K + PAD, lane);
                a = mma_bf16(frag(&u1.kq.kn[16 * wv][kk], K + PAD, lane), kj, a);
                pt = mma_bf16(kj, frag(&u1.kq.qn[16 * wv][kk], K + PAD, lane), pt);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * wv + 4 * (lane >> 4) + r, j = 16 * jt + (lane & 15);
                am[i][j] = (j < i) ? s_beta[i] * expf(s_gam[i] - s_gam[j]) * a[r] : 0.0f;
            }
        }
        const int i = 16 * wv + (lane & 15), j = 16 * jt + 4 * (lane >> 4);
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = (j + r <= i) ? expf(s_gam[i] - s_gam[j + r]) * pt[r] : 0.0f;
        *reinterpret_cast<u32x2*>(pout + (size_t)i * CH + j) = pack4(pv[0], pv[1], pv[2], pv[3]);
    }
    __syncthreads();  // A ready; kn and qn dead (tm may be written)

    // T = (I + A)^{-1}.  Diagonal 16x16 blocks by forward substitution (wave w, lanes 0..15 own the
    // columns of block w); T is zero above the diagonal.
    for (int idx = tid; idx < CH * CH; idx += 256) u1.tm[idx / CH][idx % CH] = 0.0f;
    __syncthreads();
    if (lane < 16) {
        const int c = lane, o = 16 * wv;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v = (i == c) ? 1.0f : 0.0f;
#pragma unroll
            for (int m = 0; m < i; ++m) v = fmaf(-am[o + i][o + m], x[m], v);
            x[i] = v;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) u1.tm[o + i][o + c] = x[i];
    }
    __syncthreads();
    // Off-diagonal blocks, one block diagonal at a time: T_ij = -T_ii sum_{j<=m<i} A_im T_mj.
    for (int d = 1; d < 4; ++d) {
        const int bj = wv, bi = wv + d;
        const bool act = bi < 4;
        if (act) {
            f32x4 y = zero4();
            for (int m = bj; m < bi; ++m)
#pragma unroll
                for (int kk = 0; kk < 16; kk += 4)
                    y = mma_f32(am[16 * bi + (lane & 15)][16 * m + kk + (lane >> 4)],
                                u1.tm[16 * m + kk + (lane >> 4)][16 * bj + (lane & 15)], y);
#pragma unroll
            for (int r = 0; r < 4; ++r) scr[wv][4 * (lane >> 4) + r][lane & 15] = y[r];
        }
        __syncthreads();
        if (act) {
            f32x4 z = zero4();
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4)
                z = mma_f32(u1.tm[16 * bi + (lane & 15)][16 * bi + kk + (lane >> 4)], scr[wv][kk + (lane >> 4)][lane & 15], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) u1.tm[16 * bi + 4 * (lane >> 4) + r][16 * bj + (lane & 15)] = -z[r];
        }
        __syncthreads();
    }
    // T to bf16 (overwrites A, which is dead)
    for (int idx = tid; idx < CH * CH; idx += 256) {
        const int i = idx / CH, j = idx % CH;
        tb[i][j] = bf(u1.tm[i][j]);
    }
    __syncthreads();  // tm dead: Y^T may be staged in its place
    {
        const float bi = s_beta[ti];
#pragma unroll
        for (int e = 0; e < VPT; ++e) u1.yt[part * VPT + e][ti] = bf(bi * vv[e]);
    }
    __syncthreads();

    // W^T = X^T T^T  ->  lane writes W[i][k..k+3]
    uint16_t* wout = reinterpret_cast<uint16_t*>(p.ws + p.L.w) + chh * CH * K;
    for (int tile = wv; tile < (K / 16) * 4; tile += 4) {
        const int kt = tile >> 2, it = tile & 3;
        f32x4 acc = zero4();
#pragma unroll
        for (int jj = 0; jj < CH; jj += 32) acc = mma_bf16(frag(&xt[16 * kt][jj], CH + PAD, lane), frag(&tb[16 * it][jj], CH + PAD, lane), acc);
        const int i = 16 * it + (lane & 15), k = 16 * kt + 4 * (lane >> 4);
        *reinterpret_cast<u32x2*>(wout + (size_t)i * K + k) = pack4(acc[0], acc[1], acc[2], acc[3]);
    }
    // U' = T Y  ->  lane writes U'^T[v][i..i+3]
    uint16_t* upt = reinterpret_cast<uint16_t*>(p.ws + p.L.upt) + chh * V * CH;
    for (int tile = wv; tile < 4 * (V / 16); tile += 4) {
        const int it = tile / (V / 16), vt = tile % (V / 16);
        f32x4 acc = zero4();
#pragma unroll
        for (int jj = 0; jj < CH; jj += 32) acc = mma_bf16(frag(&tb[16 * it][jj], CH + PAD, lane), frag(&u1.yt[16 * vt][jj], CH + PAD, lane), acc);
        const int v = 16 * vt + (lane & 15), i = 16 * it + 4 * (lane >> 4);
        *reinterpret_cast<u32x2*>(upt + (size_t)v * CH + i) = pack4(acc[0], acc[1], acc[2], acc[3]);
    }
}

// Operands of one chunk as one lane reads them.  Two of each alternate (ping-pong): while one chunk
// is processed the next chunk's loads are in flight, and nothing is derived from a fetched value
// until it is used, so no wait is forced early.  State waves use StateFrags, output waves OutFrags.
template <int K, int NCT>
struct StateFrags {
    bf16x8 w[K / 32];          // W rows of this wave's token tile
    u32x2 up[NCT];             // U'^T[v][4 tokens] per column tile
    bf16x8 kd[K / 64][2];      // Kd^T rows of this wave's k tiles
    float gC;                  // G_C
};
template <int K>
struct OutFrags {
    bf16x8 q[K / 32];          // raw q rows of this wave's token tile (bf16)
    bf16x8 pm[2];              // P rows of this wave's token tile
    float gi, rq;              // G_i and 1/|q_i| of this lane's output token
};

// ---- state + output ---------------------------------------------------------------------------------
// One block of 8 waves per (sequence, head, VT-column tile; VT = 16 NCT).  Loads of the chunk's
// W, Kd, q and P are shared by the block's NCT 16-column tiles.
//   Waves 0-3 ("state") carry the serial chain for chunk c: the entering state -> LDS (bf16),
//   U = U' - W S^T for token tile w, and S^T <- e^{G_C} S^T + Kd^T U for k tiles of wave w.  The state
//   is held transposed (accumulator lane: 4 consecutive k of one value column), which makes its LDS
//   copy and its HBM load/store contiguous.
//   Waves 4-7 ("output") compute chunk c-1's output O^T[v][i] = rq_i e^{G_i} (S q_i) + (U^T P^T)[v][i]
//   for token tile w from the double-buffered S and U^T, off the serial chain.
template <typename T, int K, int V, int NCT>
__global__ __launch_bounds__(512) void chunk_state_kernel(ChunkArgs p) {
    using TS = typename T::storage;
    constexpr int VT = 16 * NCT;
    constexpr int KTW = K / 64;  // 16-wide k tiles per state wave
    static_assert(V % VT == 0, "column tiles");
    __shared__ __align__(16) uint16_t sb[2][VT][K + PAD];   // S entering the chunk (bf16)
    __shared__ __align__(16) uint16_t ut[2][VT][CH + PAD];  // U^T (bf16)

    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.ws + p.L.hdr);
    if (hdr[0] != GDN_OK) return;
    const int32_t* cstart = hdr + 16;
    constexpr int NVT = V / VT;
    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, NVT);
    const int vt = blk % NVT;
    const int bh = blk / NVT;
    const int h = bh % p.H, b = bh / p.H;
    const int kh = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63;
    const bool is_state = tid < 256;
    const int wv = (tid >> 6) & 3;  // token / k tile of this wave within its group
    const int v0 = vt * VT;
    const size_t col0 = ((size_t)b * p.H + h) * V + v0;  // first state row of the block
    const TS* qkv = static_cast<const TS*>(p.qkv);
    TS* outp = static_cast<TS*>(p.out);
    const int c0 = cstart[b], c1 = cstart[b + 1];
    const int seq_start = p.offsets[b], seq_end = p.offsets[b + 1];
    const uint16_t* wbase = reinterpret_cast<const uint16_t*>(p.ws + p.L.w);
    const uint16_t* uptb = reinterpret_cast<const uint16_t*>(p.ws + p.L.upt);
    const uint16_t* kdtb = reinterpret_cast<const uint16_t*>(p.ws + p.L.kdt);
    const uint16_t* pmb = reinterpret_cast<const uint16_t*>(p.ws + p.L.pm);
    const float* gamb = reinterpret_cast<const float*>(p.ws + p.L.gam);
    const float* rqb = reinterpret_cast<const float*>(p.ws + p.L.rq);

    // transposed state tiles (state waves): acc[t][ct][r] = S[v0 + 16 ct + l%16][16 (KTW w + t) + 4(l/16) + r]
    f32x4 acc[KTW][NCT];
    if (is_state) {
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const size_t off = (col0 + 16 * ct + (lane & 15)) * K + 16 * (KTW * wv + t) + 4 * (lane >> 4);
                acc[t][ct] = p.state_in ? *reinterpret_cast<const f32x4*>(p.state_in + off) : zero4();
            }
    }

    auto fetch_s = [&](int c, StateFrags<K, NCT>& f) {
        const size_t chh = (size_t)c * p.H + h;
        const uint16_t* wrow = wbase + (chh * CH + 16 * wv) * K;
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk) f.w[kk] = frag(wrow + 32 * kk, K, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            f.up[ct] = *reinterpret_cast<const u32x2*>(uptb + (chh * V + v0 + 16 * ct + (lane & 15)) * CH + 16 * wv + 4 * (lane >> 4));
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) f.kd[t][jj] = frag(kdtb + (chh * K + 16 * (KTW * wv + t)) * CH + 32 * jj, CH, lane);
        f.gC = gamb[chh * CH + CH - 1];
    };
    auto fetch_o = [&](int c, OutFrags<K>& f) {
        const size_t chh = (size_t)c * p.H + h;
        // q rows of this lane's output token; past the sequence end the row index is clamped to the
        // sequence's last token (a valid row): those columns of the tile are never stored
        const int tq = min(seq_start + (c - c0) * CH + 16 * wv + (lane & 15), seq_end - 1);
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk) {
            if constexpr (std::is_same<T, BF16>::value) {
                f.q[kk] = *reinterpret_cast<const bf16x8*>(qkv + (size_t)tq * p.C + (size_t)kh * K + 32 * kk + 8 * (lane >> 4));
            } else {
                float t8[8];
                load8<T>(qkv + (size_t)tq * p.C + (size_t)kh * K + 32 * kk + 8 * (lane >> 4), t8);
#pragma unroll
                for (int z = 0; z < 8; ++z) f.q[kk][z] = (__bf16)t8[z];
            }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) f.pm[jj] = frag(pmb + (chh * CH + 16 * wv) * CH + 32 * jj, CH, lane);
        const int io = 16 * wv + (lane & 15);
        f.gi = gamb[chh * CH + io];
        f.rq = rqb[chh * CH + io];
    };

    // state waves, before the first barrier: S entering the chunk -> LDS (one 8-byte store per tile)
    auto s_store = [&](int buf) {
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                *reinterpret_cast<u32x2*>(&sb[buf][16 * ct + (lane & 15)][16 * (KTW * wv + t) + 4 * (lane >> 4)]) =
                    pack4(acc[t][ct][0], acc[t][ct][1], acc[t][ct][2], acc[t][ct][3]);
    };
    // state waves, between the barriers: U = U' - W S^T for token tile wv.  All LDS fragments are read
    // before the first product so that the NCT accumulation chains run back to back.
    auto s_u = [&](int buf, const StateFrags<K, NCT>& f) {
        bf16x8 sf[K / 32][NCT];
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) sf[kk][ct] = frag(&sb[buf][16 * ct][32 * kk], K + PAD, lane);
        f32x4 pw[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) pw[ct] = mma_bf16(f.w[0], sf[0][ct], zero4());
#pragma unroll
        for (int kk = 1; kk < K / 32; ++kk)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) pw[ct] = mma_bf16(f.w[kk], sf[kk][ct], pw[ct]);
        order_reads_then_mfma<K / 32 * NCT, K / 32 * NCT>();
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float u0 = bf16_bits_to_f32(f.up[ct].x & 0xffffu) - pw[ct][0];
            const float u1 = bf16_bits_to_f32(f.up[ct].x >> 16) - pw[ct][1];
            const float u2 = bf16_bits_to_f32(f.up[ct].y & 0xffffu) - pw[ct][2];
            const float u3 = bf16_bits_to_f32(f.up[ct].y >> 16) - pw[ct][3];
            *reinterpret_cast<u32x2*>(&ut[buf][16 * ct + (lane & 15)][16 * wv + 4 * (lane >> 4)]) = pack4(u0, u1, u2, u3);
        }
    };
    // state waves, after the second barrier: S^T <- e^{G_C} S^T + Kd^T U
    auto s_update = [&](int buf, const StateFrags<K, NCT>& f) {
        const float gC = expf(f.gC);
        bf16x8 uf[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) uf[ct][jj] = frag(&ut[buf][16 * ct][32 * jj], CH + PAD, lane);
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = mma_bf16(f.kd[t][0], uf[ct][0], acc[t][ct] * gC);
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = mma_bf16(f.kd[t][1], uf[ct][1], acc[t][ct]);
        order_reads_then_mfma<2 * NCT, 2 * KTW * NCT>();
    };
    // output waves: chunk c's output tiles (token tile wv, all column tiles) from sb[buf], ut[buf]
    auto o_tile = [&](int c, int buf, const OutFrags<K>& f) {
        const int t = seq_start + (c - c0) * CH + 16 * wv + (lane & 15);
        const float cs = f.rq * expf(f.gi);
        bf16x8 sf[NCT][K / 32], uf[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int kk = 0; kk < K / 32; ++kk) sf[ct][kk] = frag(&sb[buf][16 * ct][32 * kk], K + PAD, lane);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) uf[ct][jj] = frag(&ut[buf][16 * ct][32 * jj], CH + PAD, lane);
        }
        f32x4 a1[NCT], a2[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            a1[ct] = mma_bf16(sf[ct][0], f.q[0], zero4());
            a2[ct] = mma_bf16(uf[ct][0], f.pm[0], zero4());
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) a2[ct] = mma_bf16(uf[ct][1], f.pm[1], a2[ct]);
#pragma unroll
        for (int kk = 1; kk < K / 32; ++kk)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) a1[ct] = mma_bf16(sf[ct][kk], f.q[kk], a1[ct]);
        order_reads_then_mfma<(K / 32 + 2) * NCT, (K / 32 + 2) * NCT>();
        if (t < seq_end) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = p.scale * fmaf(cs, a1[ct][r], a2[ct][r]);
                TS* dst = outp + ((size_t)t * p.H + h) * V + v0 + 16 * ct + 4 * (lane >> 4);
                *reinterpret_cast<u32x2*>(dst) = u32x2{(uint32_t)from_f32<T>(o[0]) | ((uint32_t)from_f32<T>(o[1]) << 16),
                                                       (uint32_t)from_f32<T>(o[2]) | ((uint32_t)from_f32<T>(o[3]) << 16)};
            }
        }
    };

    // Iteration c (c0 <= c <= c1): state waves process chunk c (when c < c1), output waves chunk c-1
    // (when c > c0).  Every fetch is unconditional (chunk indices clamped into [c0, c1)), so the loads
    // in flight are the same on every path and each wait covers only the data about to be used.
    if (c0 < c1) {
        if (is_state) {
            StateFrags<K, NCT> fa, fb;
            fetch_s(c0, fa);
            for (int c = c0; c <= c1; c += 2) {
                fetch_s(min(c + 1, c1 - 1), fb);
                if (c < c1) s_store((c - c0) & 1);
                __syncthreads();
                if (c < c1) s_u((c - c0) & 1, fa);
                __syncthreads();
                if (c < c1) s_update((c - c0) & 1, fa);
                if (c + 1 > c1) break;
                fetch_s(min(c + 2, c1 - 1), fa);
                if (c + 1 < c1) s_store((c + 1 - c0) & 1);
                __syncthreads();
                if (c + 1 < c1) s_u((c + 1 - c0) & 1, fb);
                __syncthreads();
                if (c + 1 < c1) s_update((c + 1 - c0) & 1, fb);
            }
        } else {
            // chunk j's operands live in fa (j - c0 even) or fb (odd): fetched in iteration j, used in
            // iteration j + 1
            OutFrags<K> fa, fb;
            for (int c = c0; c <= c1; c += 2) {
                fetch_o(min(c, c1 - 1), fa);
                __syncthreads();
                if (c > c0) o_tile(c - 1, (c - 1 - c0) & 1, fb);
                __syncthreads();
                if (c + 1 > c1) break;
                fetch_o(min(c + 1, c1 - 1), fb);
                __syncthreads();
                o_tile(c, (c - c0) & 1, fa);
                __syncthreads();
            }
        }
    }
    if (is_state && p.state_out != nullptr) {
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const size_t off = (col0 + 16 * ct + (lane & 15)) * K + 16 * (KTW * wv + t) + 4 * (lane >> 4);
                *reinterpret_cast<f32x4*>(p.state_out + off) = acc[t][ct];
            }
    }
}

template <typename T, int K, int V>
hipError_t launch_kv(ChunkArgs p, hipStream_t stream) {
    const long long nch = ((long long)p.N + CH - 1) / CH + p.B;
    const long long par_blocks = nch * p.H;
    // Column tile of the state kernel: 64 columns share one load of the chunk's operands, 16 columns
    // give four times the blocks.  Wide tiles win once they still fill every compute unit.
    const long long wide_blocks = (long long)p.B * p.H * (V / 64);
    const bool wide = wide_blocks >= 256;
    const long long seq_blocks = wide ? wide_blocks : (long long)p.B * p.H * (V / 16);
    if (par_blocks > kMaxBlocks || seq_blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(1024), 0, stream, p);
    p.n_blocks = (int)par_blocks;
    hipLaunchKernelGGL((chunk_prep_kernel<T, K, V>), dim3((unsigned)par_blocks), dim3(256), 0, stream, p);
    p.n_blocks = (int)seq_blocks;
    if (wide)
        hipLaunchKernelGGL((chunk_state_kernel<T, K, V, 4>), dim3((unsigned)seq_blocks), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((chunk_state_kernel<T, K, V, 1>), dim3((unsigned)seq_blocks), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ChunkArgs& p, hipStream_t stream) {
    if (p.K == 128 && p.V == 128) return launch_kv<T, 128, 128>(p, stream);
    if (p.K == 64 && p.V == 64) return launch_kv<T, 64, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

bool chunked_shape_supported(int K, int V, int qkv_dtype) {
    return (qkv_dtype == GDN_BF16 || qkv_dtype == GDN_F16) && ((K == 128 && V == 128) || (K == 64 && V == 64));
}

size_t chunked_workspace_bytes(int B, int N, int HQ, int H, int K, int V) {
    (void)HQ;
    return ws_layout(B, N, H, K, V).total;
}

hipError_t launch_scan_chunked(const ScanLaunch& a, hipStream_t stream) {
    ChunkArgs p;
    p.qkv = a.qkv;
    p.a = a.a;
    p.b = a.b;
    p.A_log = a.A_log;
    p.dt_bias = a.dt_bias;
    p.state_in = a.state_in;
    p.out = a.out;
    p.state_out = a.state_out;
    p.offsets = a.offsets;
    p.dev_status = a.dev_status;
    p.ws = static_cast<char*>(a.workspace);
    p.L = ws_layout(a.B, a.N, a.H, a.K, a.V);
    p.B = a.B;
    p.N = a.N;
    p.HQ = a.HQ;
    p.H = a.H;
    p.K = a.K;
    p.V = a.V;
    p.C = 2 * a.HQ * a.K + a.H * a.V;
    p.G = a.H / a.HQ;
    p.gate_dtype = a.gate_dtype;
    p.flags = a.flags;
    p.scale = a.scale;
    p.n_blocks = 0;
    if (a.qkv_dtype == GDN_BF16) return launch_t<BF16>(p, stream);
    if (a.qkv_dtype == GDN_F16) return launch_t<F16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
