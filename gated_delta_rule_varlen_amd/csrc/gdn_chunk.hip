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
//          builds the table of each sequence's first chunk and an order of the sequences by
//          decreasing chunk count.
//   prep   one block per (chunk, head), parallel: gates, G, the normalised q and k, A and the masked
//          Q K^T by MFMA, T by blocked inversion (16x16 diagonal blocks by substitution, off-diagonal
//          blocks by fp32 MFMA), W^T = X^T T^T and U' = T Y by MFMA.  Writes W, P = M o (Qhat Khat^T),
//          U' and G per (chunk, value head), and Qhat and Khat^T once per (chunk, key head): they do
//          not depend on the decay, so the G value heads of a key head share them.
//   state  one block per (sequence, head, column tile), sequential over the sequence's chunks:
//          U = U' - W S^T, S <- e^{G_C} S + (diag(e^{G_C - G}) U)^T Khat, with the fp32 state in
//          MFMA accumulators; the output of the previous chunk from the same LDS copies of S and U
//          on separate waves.
//
// Every MFMA operand the state kernel reads from the workspace is stored in fragment order: the
// 16 x 32 bf16 block one instruction consumes is 64 consecutive 16-byte pieces, lane l's piece at
// 16 l (operand lane layout of v_mfma_f32_16x16x32_bf16: lane l holds row l%16, inner elements
// 8*(l/16)..+7; accumulator lane l holds rows 4*(l/16)..+3 of column l%16).  A wave then loads a
// fragment as one contiguous 1 KB access: a row-major fragment touches sixteen 128-byte lines per
// instruction, and on gfx950 that pattern moves about a third of the bytes per clock per compute unit
// that a contiguous one does.
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

// Fragment tiles.  An A tile is one 16 x 32 bf16 operand block in lane order (lane l: row l%16,
// inner elements 8(l/16)..+7; 512 elements).  A D tile is one 16 x 16 block in accumulator order
// (lane l: rows 4(l/16)..+3 of column l%16; 256 elements).
constexpr int AT = 512;
constexpr int DT = 256;

// Workspace layout (byte offsets), identical on host and device.  Per (chunk, value head) "chh",
// or per (chunk, key head) "chk" where marked:
struct WsLayout {
    size_t hdr;      // int32: [0] status, [1] total chunks; cstart[B+1] at +64, then order[B]
    size_t w;        // W      (CH x K, rows = tokens):      A tiles [4][K/32]
    size_t kt;       // Khat^T (K x CH, rows = keys):        A tiles [K/16][2]        (chk)
    size_t qf;       // Qhat   (CH x K, rows = tokens):      A tiles [4][K/32]        (chk)
    size_t pm;       // P      (CH x CH, rows = tokens i):   A tiles [4][2], P = M o (Qhat Khat^T)
    size_t upt;      // U'     (CH x V):                     D tiles [4][V/16]
    size_t gam;      // G      [CH] f32
    size_t total;
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline WsLayout ws_layout(int B, int N, int HQ, int H, int K, int V) {
    WsLayout L;
    const size_t nch = ((size_t)N + CH - 1) / CH + (size_t)B;  // upper bound on chunks over all sequences
    const size_t nh = nch * (size_t)H, nk = nch * (size_t)HQ;
    size_t o = 0;
    L.hdr = o;
    o = align256(o + 64 + 4 * (2 * (size_t)B + 1));
    L.w = o;
    o = align256(o + nh * CH * K * 2);
    L.kt = o;
    o = align256(o + nk * K * CH * 2);
    L.qf = o;
    o = align256(o + nk * CH * K * 2);
    L.pm = o;
    o = align256(o + nh * CH * CH * 2);
    L.upt = o;
    o = align256(o + nh * CH * V * 2);
    L.gam = o;
    o = align256(o + nh * CH * 4);
    L.total = o;
    return L;
}

// Half of an A tile's lane piece from an accumulator: an accumulator lane holding rows 4(l/16)..+3
// of column l%16 of the 16 x 16 block at inner offset 16*half of a 32-wide A tile writes elements
// [4(l/16) + 16 half, +4) of row l%16, which is lane piece (l%16) + 16*(2 half + (l/16)/2) at
// element 4*((l/16)%2).  Returns the element offset inside the tile.
__device__ __forceinline__ int a_tile_half_offset(int lane, int half) {
    const int g = lane >> 4;
    return ((lane & 15) + 16 * (2 * half + (g >> 1))) * 8 + 4 * (g & 1);
}

struct ChunkArgs {
    TokenStreams x;
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
    int B, N, HQ, H, K, V, G;
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
    // The state kernel's blocks are long-lived and can outnumber the blocks resident at once, so
    // they take the sequences longest first (list scheduling: the critical path is then close to the
    // longest sequence rather than a late start plus it).  Up to 1024 sequences are ranked here;
    // beyond that the order is the identity.
    int32_t* order = cstart + p.B + 1;
    __shared__ int s_cnt[1024];
    if (p.B <= 1024) {
        const int i = threadIdx.x;
        if (i < p.B) s_cnt[i] = (p.offsets[i + 1] - p.offsets[i] + CH - 1) / CH;
        __syncthreads();
        if (i < p.B) {
            const int ci = s_cnt[i];
            int rank = 0;
            for (int j = 0; j < p.B; ++j) {
                const int cj = s_cnt[j];
                rank += (cj > ci) || (cj == ci && j < i);
            }
            order[rank] = i;
        }
    } else {
        for (int i = threadIdx.x; i < p.B; i += blockDim.x) order[i] = i;
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

// Eight 16-bit values packed in 16 bytes -> fp32.
template <typename T>
__device__ __forceinline__ void unpack8(u32x4 raw, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = to_f32<T>((uint16_t)(raw[e] & 0xffffu));
        v[2 * e + 1] = to_f32<T>((uint16_t)(raw[e] >> 16));
    }
}

__device__ __forceinline__ u32x4 pack8(const float* x, float s) {
    return u32x4{(uint32_t)bf(x[0] * s) | ((uint32_t)bf(x[1] * s) << 16), (uint32_t)bf(x[2] * s) | ((uint32_t)bf(x[3] * s) << 16),
                 (uint32_t)bf(x[4] * s) | ((uint32_t)bf(x[5] * s) << 16), (uint32_t)bf(x[6] * s) | ((uint32_t)bf(x[7] * s) << 16)};
}

// ---- prep ----------------------------------------------------------------------------------------
// k and v token rows are read whole: LPT = K/8 lanes per row, 8 elements (16 bytes) each, so one
// wave instruction covers 64/LPT complete rows.  Column operands (8 consecutive tokens of one key or
// value index) are gathered from the row-major LDS copies with 2-byte reads.  A wave needs only its
// own 16 rows of Qhat, as MFMA fragments: they are loaded in fragment order and stay in registers.
// LDS is shared by lifetime (39 KB at K = 128, so four blocks fit on a compute unit):
//   region 0: Khat rows, until A and P are formed; then T (fp32)
//   region 2: Y rows, until their fragments are in registers; then A (fp32); then T (bf16)
//   the off-diagonal inversion scratch has its own 4 KB
template <typename T, int K, int V>
__global__ __launch_bounds__(256, 4) void chunk_prep_kernel(ChunkArgs p) {
    using TS = typename T::storage;
    static_assert(K == V && (K == 64 || K == 128), "chunk tile shapes");
    constexpr int LPT = K / 8;     // lanes per token row
    constexpr int TPI = 64 / LPT;  // token rows per wave instruction
    constexpr int NI = 16 / TPI;   // instructions per wave for its 16 rows
    constexpr int KT4 = K / 64;    // 16-wide key (value) tiles per wave
    __shared__ __align__(16) union {
        uint16_t kn[CH][K + PAD];  // Khat rows
        float tm[CH][CH + 4];      // T (fp32)
    } r0;
    __shared__ float scr[4][16][17];  // off-diagonal inversion scratch
    __shared__ __align__(16) union {
        uint16_t vn[CH][V + PAD];  // Y = diag(b) V rows
        float am[CH][CH + 4];      // A (fp32)
        uint16_t tb[CH][CH + PAD];  // T (bf16)
    } r2;
    __shared__ __align__(16) float s_gam[CH], s_beta[CH], s_xs[CH];
    auto& kn = r0.kn;
    auto& tm = r0.tm;
    auto& vn = r2.vn;
    auto& am = r2.am;
    auto& tb = r2.tb;

    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.ws + p.L.hdr);
    if (hdr[0] != GDN_OK) return;
    const int total = hdr[1];
    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, p.G);
    // Chunks are taken last first: the operands written last are the likeliest still to sit in the
    // 256 MB memory-side cache when the state kernel starts, and it starts from the first chunks
    // (one long sequence: 1477 -> 1429 us for the whole call).
    const int cid = p.n_blocks / p.H - 1 - blk / p.H, h = blk % p.H;
    if (cid >= total) return;
    const int32_t* cstart = hdr + 16;
    const int b = chunk_owner(cstart, p.B, cid);
    const int t0 = p.offsets[b] + (cid - cstart[b]) * CH;
    const int n = min(CH, p.offsets[b + 1] - t0);
    const int kh = h / p.G;
    const size_t chh = (size_t)cid * p.H + h;
    const size_t chk = (size_t)cid * p.HQ + kh;
    // Qhat and Khat^T are the same for every value head of the key head: the first one writes them
    const bool shared_writer = (h % p.G) == 0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int pc = lane % LPT, tsub = lane / LPT;
    const TS* const xq = static_cast<const TS*>(p.x.q);
    const TS* const xk = static_cast<const TS*>(p.x.k);
    const TS* const xv = static_cast<const TS*>(p.x.v);
    uint16_t* const wsb = reinterpret_cast<uint16_t*>(p.ws);
    uint16_t* const w_out = wsb + p.L.w / 2 + chh * CH * K;
    uint16_t* const kt_out = wsb + p.L.kt / 2 + chk * K * CH;
    uint16_t* const q_out = wsb + p.L.qf / 2 + chk * CH * K;
    uint16_t* const p_out = wsb + p.L.pm / 2 + chh * CH * CH;
    uint16_t* const u_out = wsb + p.L.upt / 2 + chh * CH * V;

    // this wave's 16 token rows (row 16 wv + TPI u + tsub), elements 8 pc .. 8 pc + 7, kept packed
    // (16-bit inputs) until the gates are known
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int ti = 16 * wv + TPI * u + tsub;
        if (ti < n) {
            const size_t t = (size_t)(t0 + ti);
            kr[u] = *reinterpret_cast<const u32x4*>(xk + t * p.x.sk + (size_t)kh * K + 8 * pc);
            vr[u] = *reinterpret_cast<const u32x4*>(xv + t * p.x.sv + (size_t)h * V + 8 * pc);
        } else {
            kr[u] = vr[u] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // this wave's q rows in MFMA operand order: lane l holds row 16 wv + l%16, elements
    // 32 kk + 8(l/16) .. +7 of fragment kk
    u32x4 qr[K / 32];
    {
        const int ti = 16 * wv + (lane & 15);
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk)
            qr[kk] = ti < n ? *reinterpret_cast<const u32x4*>(xq + (size_t)(t0 + ti) * p.x.sq + (size_t)kh * K + 32 * kk +
                                                              8 * (lane >> 4))
                            : u32x4{0u, 0u, 0u, 0u};
    }

    // gates and the cumulative log-decay (wave 0, one token per lane); padding tokens have b = 0
    // and no decay
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
        s_xs[lane] = beta * expf(gam);
        reinterpret_cast<float*>(p.ws + p.L.gam)[chh * CH + lane] = gam;
    }
    __syncthreads();  // gates ready

    // normalised k rows and Y = diag(b) V rows -> LDS
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int ti = 16 * wv + TPI * u + tsub;
        float kf[8], vf[8];
        unpack8<T>(kr[u], kf);
        unpack8<T>(vr[u], vf);
        float sk = 0.0f;
#pragma unroll
        for (int z = 0; z < 8; ++z) sk = fmaf(kf[z], kf[z], sk);
        sk = group_sum<LPT>(sk);
        *reinterpret_cast<u32x4*>(&kn[ti][8 * pc]) = pack8(kf, rsqrtf(sk + 1e-12f));
        *reinterpret_cast<u32x4*>(&vn[ti][8 * pc]) = pack8(vf, s_beta[ti]);
    }
    // normalised q fragments (the four lanes l%16 + 16 j hold one row between them)
    bf16x8 qw[K / 32];
    {
        float qf[K / 32][8];
        float sq = 0.0f;
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk) {
            unpack8<T>(qr[kk], qf[kk]);
#pragma unroll
            for (int z = 0; z < 8; ++z) sq = fmaf(qf[kk][z], qf[kk][z], sq);
        }
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        const float rq = rsqrtf(sq + 1e-12f);
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk) {
            u32x4 pq = pack8(qf[kk], rq);
            asm volatile("" : "+v"(pq));  // pack now (see the column fragments below)
            qw[kk] = __builtin_bit_cast(bf16x8, pq);
        }
    }
    __syncthreads();  // kn, vn ready

    // Qhat tiles (token tile wv)
    if (shared_writer) {
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk)
            *reinterpret_cast<bf16x8*>(q_out + (size_t)(wv * (K / 32) + kk) * AT + 8 * lane) = qw[kk];
    }

    // Column fragments of key tiles kt = wv + 4m: Khat^T (stored) and X^T = (diag(b e^G) Khat)^T (kept
    // for W), and of value tiles vt = wv + 4m: Y (kept for U').  Lane l: index 16 kt + l%16, tokens
    // 32 c + 8(l/16) + e.
    bf16x8 xf[KT4][2], yf[KT4][2];
#pragma unroll
    for (int m = 0; m < KT4; ++m) {
        const int kt = wv + 4 * m, col = 16 * kt + (lane & 15);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int tb0 = 32 * c + 8 * (lane >> 4);
            float kx[8];
            u32x4 kc, yp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t k0 = kn[tb0 + 2 * e][col], k1 = kn[tb0 + 2 * e + 1][col];
                kx[2 * e] = s_xs[tb0 + 2 * e] * bf16_bits_to_f32(k0);
                kx[2 * e + 1] = s_xs[tb0 + 2 * e + 1] * bf16_bits_to_f32(k1);
                kc[e] = (uint32_t)k0 | ((uint32_t)k1 << 16);
                yp[e] = (uint32_t)vn[tb0 + 2 * e][col] | ((uint32_t)vn[tb0 + 2 * e + 1][col] << 16);
            }
            if (shared_writer) *reinterpret_cast<u32x4*>(kt_out + (size_t)(kt * 2 + c) * AT + 8 * lane) = kc;
            u32x4 xp = pack8(kx, 1.0f);
            // Pack here: left to itself the compiler keeps the eight 16-bit values of a fragment in
            // eight registers until the products far below, which spills.  The empty statements
            // (no instructions) pin the packed values at this point.
            asm volatile("" : "+v"(xp));
            asm volatile("" : "+v"(yp));
            xf[m][c] = __builtin_bit_cast(bf16x8, xp);
            yf[m][c] = __builtin_bit_cast(bf16x8, yp);
        }
    }

    __syncthreads();  // Y gathered: A may overwrite it

    // A_ij = b_i e^{G_i - G_j} (khat_i . khat_j) for j < i, and P_ij = e^{G_i - G_j} (qhat_i . khat_j)
    // for j <= i, in 16 x 16 blocks.  Wave wv forms the P blocks of its own row tile (it holds those
    // Qhat rows; computed transposed: 4 consecutive j per lane) and the A blocks of column tile wv
    // (rows it..3), so that every wave does 5 of the 20 nonzero blocks.  The masks are selects, not
    // branches: the decay factor is evaluated for every entry with its exponent clamped at 0 (G never
    // increases inside a chunk, so the clamp changes only entries the mask drops), and G and b are
    // read as 4-vectors.  The tile loops stay rolled: the X and Y fragments are live across them,
    // and unrolled they need more registers than four blocks per compute unit leave.
    {
        const int ip = 16 * wv + (lane & 15);  // row of this lane's P entries
#pragma unroll 1
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 pt = zero4();
            if (jt <= wv) {
#pragma unroll
                for (int kk = 0; kk < K; kk += 32) pt = mma_bf16(frag(&kn[16 * jt][kk], K + PAD, lane), qw[kk / 32], pt);
            }
            const int j = 16 * jt + 4 * (lane >> 4);
            const f32x4 g_j = *reinterpret_cast<const f32x4*>(&s_gam[j]);
            const float g_ip = s_gam[ip];
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = expf(fminf(g_ip - g_j[r], 0.0f));
                pv[r] = (j + r <= ip) ? e * pt[r] : 0.0f;
            }
            // (token tiles 0 and 1 have no nonzero entry past key 31; that fragment is never read)
            if (wv >= 2 || jt < 2)
                *reinterpret_cast<u32x2*>(p_out + (size_t)(wv * 2 + (jt >> 1)) * AT + a_tile_half_offset(lane, jt & 1)) =
                    pack4(pv[0], pv[1], pv[2], pv[3]);
        }
        const int ja = 16 * wv + (lane & 15);  // column of this lane's A entries
        const float g_ja = s_gam[ja];
#pragma unroll 1
        for (int it = wv; it < 4; ++it) {
            f32x4 a = zero4();
#pragma unroll
            for (int kk = 0; kk < K; kk += 32)
                a = mma_bf16(frag(&kn[16 * it][kk], K + PAD, lane), frag(&kn[16 * wv][kk], K + PAD, lane), a);
            const int ia = 16 * it + 4 * (lane >> 4);  // rows of this lane's A entries
            const f32x4 g_ia = *reinterpret_cast<const f32x4*>(&s_gam[ia]);
            const f32x4 b_ia = *reinterpret_cast<const f32x4*>(&s_beta[ia]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = expf(fminf(g_ia[r] - g_ja, 0.0f));
                am[ia + r][ja] = (ja < ia + r) ? b_ia[r] * e * a[r] : 0.0f;
            }
        }
    }
    __syncthreads();  // A ready; Khat rows dead (T may be written)

    // T = (I + A)^{-1}.  Diagonal 16x16 blocks by forward substitution (wave w, lanes 0..15 own the
    // columns of block w); T is zero above the diagonal.
    // (thread t clears 16 consecutive entries of row t/4 with 16-byte stores)
    static_assert(CH * CH == 256 * 16, "one 16-entry run per thread");
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4*>(&tm[tid >> 2][16 * (tid & 3) + 4 * q]) = zero4();
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
        for (int i = 0; i < 16; ++i) tm[o + i][o + c] = x[i];
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
                                tm[16 * m + kk + (lane >> 4)][16 * bj + (lane & 15)], y);
#pragma unroll
            for (int r = 0; r < 4; ++r) scr[wv][4 * (lane >> 4) + r][lane & 15] = y[r];
        }
        __syncthreads();
        if (act) {
            f32x4 z = zero4();
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4)
                z = mma_f32(tm[16 * bi + (lane & 15)][16 * bi + kk + (lane >> 4)], scr[wv][kk + (lane >> 4)][lane & 15], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) tm[16 * bi + 4 * (lane >> 4) + r][16 * bj + (lane & 15)] = -z[r];
        }
        __syncthreads();
    }
    // T to bf16 (overwrites A, which is dead)
    {
        // thread t converts 16 consecutive entries of row t/4: four 16-byte reads, two 16-byte writes
        const int i = tid >> 2, j0 = 16 * (tid & 3);
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&tm[i][j0 + 4 * q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
        }
        *reinterpret_cast<u32x4*>(&tb[i][j0]) = pack8(v, 1.0f);
        *reinterpret_cast<u32x4*>(&tb[i][j0 + 8]) = pack8(v + 8, 1.0f);
    }
    __syncthreads();

    // W^T = X^T T^T for key tiles kt = wv + 4m: lane holds W[i][k..k+3], half of a W tile piece
#pragma unroll
    for (int m = 0; m < KT4; ++m) {
        const int kt = wv + 4 * m;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            // T is lower triangular: rows i < 32 have no entry at j >= 32
            f32x4 acc = mma_bf16(xf[m][0], frag(&tb[16 * it][0], CH + PAD, lane), zero4());
            if (it >= 2) acc = mma_bf16(xf[m][1], frag(&tb[16 * it][32], CH + PAD, lane), acc);
            *reinterpret_cast<u32x2*>(w_out + (size_t)(it * (K / 32) + (kt >> 1)) * AT + a_tile_half_offset(lane, kt & 1)) =
                pack4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
    // U' = T Y for value tiles vt = wv + 4m: accumulator order is the D tile order
#pragma unroll
    for (int m = 0; m < KT4; ++m) {
        const int vt = wv + 4 * m;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            f32x4 acc = mma_bf16(frag(&tb[16 * it][0], CH + PAD, lane), yf[m][0], zero4());
            if (it >= 2) acc = mma_bf16(frag(&tb[16 * it][32], CH + PAD, lane), yf[m][1], acc);
            *reinterpret_cast<u32x2*>(u_out + (size_t)(it * (V / 16) + vt) * DT + 4 * lane) = pack4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

// Operands of one chunk as one lane reads them.  Two of each alternate (ping-pong): while one chunk
// is processed the next chunk's loads are in flight, and nothing is derived from a fetched value
// until it is used, so no wait is forced early.  State waves use StateFrags, output waves OutFrags.
template <int K, int NCT>
struct StateFrags {
    bf16x8 w[K / 32];          // W tiles of this wave's token tile
    u32x2 up[NCT];             // U' D-tile pieces, one per column tile
    bf16x8 kt[K / 64][2];      // Khat^T tiles of this wave's key tiles
    f32x4 gr;                  // G of this lane's four U rows (tokens 16 w + 4(l/16) .. +3)
    float gC;                  // G_C
};
template <int K>
struct OutFrags {
    bf16x8 q[K / 32];          // Qhat tiles of this wave's token tile
    bf16x8 pm[2];              // P tiles of this wave's token tile
    float gi;                  // G_i of this lane's output token
};

// ---- state + output ---------------------------------------------------------------------------------
// One block of 8 waves per (sequence, head, VT-column tile; VT = 16 NCT).  Loads of the chunk's
// W, Khat^T, Qhat and P are shared by the block's NCT 16-column tiles.
//   Waves 0-3 ("state") carry the serial chain for chunk c: the entering state -> LDS (bf16),
//   U = U' - W S^T for token tile w (to LDS as is, for the output, and with row i scaled by
//   e^{G_C - G_i} <= 1, for the update), and S^T <- e^{G_C} S^T + Khat^T Ud for key tiles of wave w.
//   The state is held transposed (accumulator lane: 4 consecutive keys of one value column), which
//   makes its LDS copy and its HBM load/store contiguous.
//   Waves 4-7 ("output") compute chunk c's output O^T[v][i] = e^{G_i} (S qhat_i) + (U^T P^T)[v][i]
//   for token tile w from the double-buffered S and U^T while the state waves update S, off the
//   serial chain, and write it as whole token rows through a per-wave LDS tile.
template <typename T, int K, int V, int NCT>
__global__ __launch_bounds__(512) void chunk_state_kernel(ChunkArgs p) {
    using TS = typename T::storage;
    constexpr int VT = 16 * NCT;
    constexpr int KTW = K / 64;  // 16-wide key tiles per state wave
    static_assert(V % VT == 0, "column tiles");
    __shared__ __align__(16) uint16_t sb[2][VT][K + PAD];   // S entering the chunk (bf16)
    __shared__ __align__(16) uint16_t ut[2][VT][CH + PAD];  // U^T (bf16)
    __shared__ __align__(16) uint16_t ud[VT][CH + PAD];     // (diag(e^{G_C - G}) U)^T (bf16)
    __shared__ __align__(16) uint16_t ot[4][16][VT + 8];    // output rows, one tile per output wave

    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.ws + p.L.hdr);
    if (hdr[0] != GDN_OK) return;
    const int32_t* cstart = hdr + 16;
    constexpr int NVT = V / VT;
    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, NVT);
    const int vt = blk % NVT;
    const int bh = blk / NVT;
    const int h = bh % p.H, b = cstart[p.B + 1 + bh / p.H];  // sequences longest first
    const int kh = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63;
    const bool is_state = tid < 256;
    const int wv = (tid >> 6) & 3;  // token / key tile of this wave within its group
    const int v0 = vt * VT;
    const size_t col0 = ((size_t)b * p.H + h) * V + v0;  // first state row of the block
    TS* outp = static_cast<TS*>(p.out);
    const int c0 = cstart[b], c1 = cstart[b + 1];
    const int seq_start = p.offsets[b], seq_end = p.offsets[b + 1];
    const uint16_t* const wsb = reinterpret_cast<const uint16_t*>(p.ws);
    const uint16_t* const wbase = wsb + p.L.w / 2;
    const uint16_t* const ktbase = wsb + p.L.kt / 2;
    const uint16_t* const qbase = wsb + p.L.qf / 2;
    const uint16_t* const pbase = wsb + p.L.pm / 2;
    const uint16_t* const ubase = wsb + p.L.upt / 2;
    const float* gamb = reinterpret_cast<const float*>(p.ws + p.L.gam);

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

    auto afrag = [&](const uint16_t* tile) { return *reinterpret_cast<const bf16x8*>(tile + 8 * lane); };
    auto fetch_s = [&](int c, StateFrags<K, NCT>& f) {
        const size_t chh = (size_t)c * p.H + h, chk = (size_t)c * p.HQ + kh;
        const uint16_t* wt = wbase + (chh * 4 + wv) * (K / 32) * AT;
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk) f.w[kk] = afrag(wt + kk * AT);
        const uint16_t* ud = ubase + ((chh * 4 + wv) * (V / 16) + vt * NCT) * DT + 4 * lane;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) f.up[ct] = *reinterpret_cast<const u32x2*>(ud + ct * DT);
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) f.kt[t][jj] = afrag(ktbase + ((chk * (K / 16) + KTW * wv + t) * 2 + jj) * AT);
        f.gr = *reinterpret_cast<const f32x4*>(gamb + chh * CH + 16 * wv + 4 * (lane >> 4));
        f.gC = gamb[chh * CH + CH - 1];
    };
    auto fetch_o = [&](int c, OutFrags<K>& f) {
        const size_t chh = (size_t)c * p.H + h, chk = (size_t)c * p.HQ + kh;
        const uint16_t* qt = qbase + (chk * 4 + wv) * (K / 32) * AT;
#pragma unroll
        for (int kk = 0; kk < K / 32; ++kk) f.q[kk] = afrag(qt + kk * AT);
        f.pm[0] = afrag(pbase + (chh * 4 + wv) * 2 * AT);
        // token tiles 0 and 1 have no nonzero P entry past key 31: that fragment is neither
        // stored nor loaded
        if (wv >= 2) f.pm[1] = afrag(pbase + ((chh * 4 + wv) * 2 + 1) * AT);
        f.gi = gamb[chh * CH + 16 * wv + (lane & 15)];
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
        float ds[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[r] = expf(f.gC - f.gr[r]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float u0 = bf16_bits_to_f32(f.up[ct].x & 0xffffu) - pw[ct][0];
            const float u1 = bf16_bits_to_f32(f.up[ct].x >> 16) - pw[ct][1];
            const float u2 = bf16_bits_to_f32(f.up[ct].y & 0xffffu) - pw[ct][2];
            const float u3 = bf16_bits_to_f32(f.up[ct].y >> 16) - pw[ct][3];
            *reinterpret_cast<u32x2*>(&ut[buf][16 * ct + (lane & 15)][16 * wv + 4 * (lane >> 4)]) = pack4(u0, u1, u2, u3);
            *reinterpret_cast<u32x2*>(&ud[16 * ct + (lane & 15)][16 * wv + 4 * (lane >> 4)]) =
                pack4(u0 * ds[0], u1 * ds[1], u2 * ds[2], u3 * ds[3]);
        }
    };
    // state waves, after the second barrier: S^T <- e^{G_C} S^T + Khat^T Ud
    auto s_update = [&](const StateFrags<K, NCT>& f) {
        const float gC = expf(f.gC);
        bf16x8 uf[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) uf[ct][jj] = frag(&ud[16 * ct][32 * jj], CH + PAD, lane);
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = mma_bf16(f.kt[t][0], uf[ct][0], acc[t][ct] * gC);
#pragma unroll
        for (int t = 0; t < KTW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = mma_bf16(f.kt[t][1], uf[ct][1], acc[t][ct]);
        order_reads_then_mfma<2 * NCT, 2 * KTW * NCT>();
    };
    // output waves: chunk c's output tiles (token tile wv, all column tiles) from sb[buf], ut[buf]
    constexpr int LPR = VT / 8;         // lanes per output row (16 bytes each)
    constexpr int RPI = 64 / LPR;       // rows per store instruction
    // NJ: the P fragments of this token tile that can be nonzero (tiles 0 and 1 see only keys < 32)
    auto o_tile = [&](auto nj, int c, int buf, const OutFrags<K>& f) {
        constexpr int NJ = decltype(nj)::value;
        const float cs = expf(f.gi);
        bf16x8 sf[NCT][K / 32], uf[NCT][NJ];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int kk = 0; kk < K / 32; ++kk) sf[ct][kk] = frag(&sb[buf][16 * ct][32 * kk], K + PAD, lane);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) uf[ct][jj] = frag(&ut[buf][16 * ct][32 * jj], CH + PAD, lane);
        }
        f32x4 a1[NCT], a2[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            a1[ct] = mma_bf16(sf[ct][0], f.q[0], zero4());
            a2[ct] = mma_bf16(uf[ct][0], f.pm[0], zero4());
        }
        if constexpr (NJ == 2) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) a2[ct] = mma_bf16(uf[ct][1], f.pm[1], a2[ct]);
        }
#pragma unroll
        for (int kk = 1; kk < K / 32; ++kk)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) a1[ct] = mma_bf16(sf[ct][kk], f.q[kk], a1[ct]);
        order_reads_then_mfma<(K / 32 + NJ) * NCT, (K / 32 + NJ) * NCT>();
        // lane: token 16 wv + l%16, columns 16 ct + 4(l/16) .. +3
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = p.scale * fmaf(cs, a1[ct][r], a2[ct][r]);
            *reinterpret_cast<u32x2*>(&ot[wv][lane & 15][16 * ct + 4 * (lane >> 4)]) =
                u32x2{(uint32_t)from_f32<T>(o[0]) | ((uint32_t)from_f32<T>(o[1]) << 16),
                      (uint32_t)from_f32<T>(o[2]) | ((uint32_t)from_f32<T>(o[3]) << 16)};
        }
        // the tile is this wave's alone: LDS keeps one wave's accesses in order, the fence keeps the
        // compiler from moving the reads above the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int tbase = seq_start + (c - c0) * CH + 16 * wv;
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += RPI) {
            const int row = r0 + lane / LPR;
            if (row < 16 && tbase + row < seq_end)
                *reinterpret_cast<u32x4*>(outp + ((size_t)(tbase + row) * p.H + h) * V + v0 + 8 * (lane % LPR)) =
                    *reinterpret_cast<const u32x4*>(&ot[wv][row][8 * (lane % LPR)]);
        }
    };

    // Iteration c (c0 <= c <= c1) has two barriers.  State waves store S entering chunk c before the
    // first, form U between them and update S after the second; output waves compute chunk c's
    // output after the second barrier (S and U of chunk c are complete then and stay untouched until
    // the next iteration's second barrier), alongside the state update.  Every fetch is
    // unconditional (chunk indices clamped into [c0, c1)), so the loads in flight are the same on
    // every path and each wait covers only the data about to be used.
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
                if (c < c1) s_update(fa);
                if (c + 1 > c1) break;
                fetch_s(min(c + 2, c1 - 1), fa);
                if (c + 1 < c1) s_store((c + 1 - c0) & 1);
                __syncthreads();
                if (c + 1 < c1) s_u((c + 1 - c0) & 1, fb);
                __syncthreads();
                if (c + 1 < c1) s_update(fb);
            }
        } else {
            // chunk j's output is computed right after the second barrier of iteration j (S entering
            // chunk j and its U are complete then), alongside the state waves' update; its operands
            // live in fa (j - c0 even) or fb (odd), fetched one iteration ahead
            OutFrags<K> fa, fb;
            fetch_o(c0, fa);
            for (int c = c0; c <= c1; c += 2) {
                __syncthreads();
                fetch_o(min(c + 1, c1 - 1), fb);
                __syncthreads();
                if (c < c1) {
                    if (wv >= 2) o_tile(std::integral_constant<int, 2>{}, c, (c - c0) & 1, fa);
                    else o_tile(std::integral_constant<int, 1>{}, c, (c - c0) & 1, fa);
                }
                if (c + 1 > c1) break;
                __syncthreads();
                fetch_o(min(c + 2, c1 - 1), fa);
                __syncthreads();
                if (c + 1 < c1) {
                    if (wv >= 2) o_tile(std::integral_constant<int, 2>{}, c + 1, (c + 1 - c0) & 1, fb);
                    else o_tile(std::integral_constant<int, 1>{}, c + 1, (c + 1 - c0) & 1, fb);
                }
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
    return ws_layout(B, N, HQ, H, K, V).total;
}

hipError_t launch_scan_chunked(const ScanLaunch& a, hipStream_t stream) {
    ChunkArgs p;
    p.x = a.x;
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
    p.L = ws_layout(a.B, a.N, a.HQ, a.H, a.K, a.V);
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
    p.n_blocks = 0;
    if (a.qkv_dtype == GDN_BF16) return launch_t<BF16>(p, stream);
    if (a.qkv_dtype == GDN_F16) return launch_t<F16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
