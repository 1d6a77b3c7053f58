// gdn_chunk.hpp -- chunked (WY / UT-transform) form of the gated delta-rule recurrence (gfx950).
//
// Operation: paged_ssm.rs page, kernel string DELTA, which the host fn delta() runs chunked for long
// prefills.  The chunked kernel's source is not on the pages, so the algebra below is derived from
// the recurrence itself.  In matrix form (S is V x K, row v = the state of value column v)
//     S_t = g_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,     o_t = scale S_t q_t.
// For one chunk of C = 64 tokens of one sequence and head, with G_i the cumulative log-decay inside
// the chunk and S0 the state entering it:
//     A_ij = b_i e^{G_i - G_j} (k_i . k_j)  (j < i),   T = (I + A)^{-1}   (unit lower triangular)
//     R    = diag(b) V - diag(b e^G) K S0^T,          U = T R             (U row i = delta_i)
//     O    = scale [ diag(e^G) Q S0^T + P U ],        P_ij = e^{G_i - G_j} (q_i . k_j) (j <= i)
//     S_C^T = e^{G_C} S0^T + K^T diag(e^{G_C - G}) U.
// Only decays that are finite and positive are allowed (log-decays are summed), which the softplus
// gate guarantees.  Chunks never cross sequence boundaries.
//
// Kernels, in stream order:
//   index    one block: checks the offsets (nothing is written anywhere when they are malformed)
//            and builds the tables (chunks per sequence, sequences longest first, segments).
//   tmat     one block per (chunk, head), fully parallel: the gates and G, A by MFMA and
//            T = (I + A)^{-1} by blocked inversion, stored as the six 16 x 32 operand fragments
//            the chain reads (6 KB), plus G, b and 1/|k| (768 B).  This is the only per-chunk
//            data that goes through memory.
//   summary  (long sequences only, below)
//   combine  (long sequences only, below)
//   main     one block per (sequence or segment, head, value part of VT <= 128 columns), serial
//            over its chunks, with one wave per 16 value columns of the part.  Each wave keeps the
//            fp32 state S0^T of its columns in MFMA accumulators.  An accumulator holds 4
//            consecutive rows of one column per lane; read as the B operand of the next product it
//            supplies inner elements in the order {4g..4g+3, 16+4g..16+4g+3} (g = lane/16) of each
//            32-block, so A operands are read in that same order ("split" fragments) and K S0^T,
//            Q S0^T, T R, P U and K^T U chain from accumulator to operand in registers.  P is formed
//            by each wave directly in that operand order.  The raw q, k and v rows of the next
//            chunk (the q and k norms scale per-token factors instead) are staged as loaded while
//            the current one is in use, and the next chunk's rows and T fragments are in flight
//            meanwhile; K^T and R's columns of v are read from the row tiles through the
//            transposing LDS read (on fp16 operands K^T is a transposed tile of normalised rows):
//            two barriers per chunk (three where LDS holds one copy of the K^T source only).
// Widths: the key width runs on the next of 64, 128 and 256 and the value width in parts of the
// next of 32, 64 and 128 columns (parts of 128 past that), with keys and columns past the real
// widths zero; loads past them read zero and stores past them are dropped.
// Long sequences with few heads leave most compute units idle, so they are cut into segments of
// seglen chunks that run in parallel (widths with one value part whose summary fits the registers).
// A segment's effect on the state is affine, S_end^T = Phi S_start^T + N^T, and its (Phi, N) come
// from the same chain run from S = 0 on the value columns (N) and from S = I on K extra columns
// with v = 0 (Phi):
//   summary  one block per (non-last segment, head): Phi and N into the workspace;
//   combine  one block per (sequence, head, 8 value rows): S_start of every segment, in order,
//            in fp32;
//   main     then runs every segment from its S_start.
#pragma once
#include <climits>
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {


constexpr int CH = kChunkTokens;  // tokens per chunk
constexpr int NW = 4;   // waves per block
// LDS rows holding MFMA operands are padded by 16 bytes so that the 16 rows a fragment read touches
// do not all start on the same banks.
// Row pitches (16-bit elements) of the LDS tiles: K + kPadRow for k/q rows, CH + kPadT for 64-token
// rows.  An odd number of 16-byte units per row makes the 16 x 16 fragment reads 2-way bank
// conflicted on gfx950; these pads give an even count and conflict-free reads.
constexpr int kPadRow = 16, kPadT = 16;
constexpr int NTF = 6;  // T fragments per chunk: (token tile, 32-block) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)

// ---- workspace ----------------------------------------------------------------------------------
// int32 header: [0] status, [1] main units, [2] summary units, [3] chunks, then the tables at +16:
//   order[B]     sequences by decreasing chunk count (rank -> sequence)
//   ustart[B+1]  first main unit of each rank (nseg * H * VS units per sequence)
//   sstart[B+1]  first summary unit of each sequence ((nseg - 1) * H units when nseg > 1)
//   slot0[B+1]   first slot of each sequence (nseg slots when nseg > 1, else none)
//   nchunk[B]    chunks of each sequence
//   cstart[B+1]  first chunk of each sequence
// Per (chunk, head): the T fragments (6 x 512 bf16, lane order) and G, b, 1/|k| (3 x 64 f32).
// Slots: per (slot, head) Phi [K][K] then N [VT][K], fp32 (a row per column, K contiguous; K and
// VT the compiled widths).  Slot
// s < nseg-1 of a sequence holds the summary of segment s, and after the combine kernel its N holds
// S_start(s+1); the N of slot nseg-1 holds S_start(0).
struct WsLayout {
    size_t hdr, tfr, gates, slots, total;
    size_t nslots;  // slots available
    int seglen;     // chunks per segment; INT_MAX = one segment per sequence
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

#ifndef GDN_CHUNK_VTW
#define GDN_CHUNK_VTW 1
#endif
constexpr int kValueTilesPerWave = GDN_CHUNK_VTW;  // 16-column value tiles per wave of the main kernel

// Compiled widths.  A key width K (a multiple of 8, at most 256) runs on the next of 64, 128 and
// 256 with the keys past K zero (they add nothing to any product and their state rows stay zero);
// a value width V (a multiple of 8) runs in value parts of VT columns, VT the next of 32, 64 and 128
// for V <= 128 and 128 past that, one block per part, with the columns past V zero.
__host__ __device__ constexpr int chunk_key_width(int K) { return K <= 64 ? 64 : K <= 128 ? 128 : 256; }
__host__ __device__ constexpr int chunk_value_tile(int V) { return V <= 32 ? 32 : V <= 64 ? 64 : 128; }
__host__ __device__ constexpr int chunk_value_parts(int V) { return V <= 128 ? 1 : (V + 127) / 128; }
// Segments need the summary form, which carries K more state columns per block (Phi): allowed when
// the value columns come in one part and a wave's share of Phi keeps its accumulators within 128
// registers (K = 64 with VT = 32 or 64, K = 128 with VT = 64 or 128).
__host__ __device__ constexpr bool chunk_segments_ok(int KP, int VT, int VS) {
    return VS == 1 && KP % (16 * (VT / (16 * kValueTilesPerWave))) == 0 &&
           (KP / 16) * (kValueTilesPerWave + KP / (16 * (VT / (16 * kValueTilesPerWave)))) <= 32;
}

// Segments are used when fewer than a quarter of the compute units would hold a (sequence, head,
// value part) unit; then each sequence is cut into about 256 / (B H) segments of at least 16 chunks.
constexpr int kChipUnits = 256;
inline long long chunk_bound(int B, int N) { return ((long long)N + CH - 1) / CH + B; }
inline int segment_length(int B, int N, int H, int K, int V) {
    const int VS = chunk_value_parts(V);
    if (!chunk_segments_ok(chunk_key_width(K), chunk_value_tile(V), VS)) return INT_MAX;
    const long long units = (long long)B * H;
    const long long per = kChipUnits / units;
    if (per < 4) return INT_MAX;
    const long long nch = chunk_bound(B, N);
    const long long avg = (nch + B - 1) / B;
    long long sl = (avg + per - 1) / per;
    if (sl < 16) sl = 16;
    return (int)sl;
}
inline WsLayout ws_layout(int B, int N, int H, int Kr, int Vr) {
    WsLayout L;
    L.seglen = segment_length(B, N, H, Kr, Vr);
    const int K = chunk_key_width(Kr), V = chunk_value_tile(Vr);  // slot widths (one value part)
    const long long nch = chunk_bound(B, N);
    L.nslots = 0;
    if (L.seglen != INT_MAX) {
        const long long multi = nch / (L.seglen + 1);  // sequences with more than one segment
        L.nslots = (size_t)(nch / L.seglen + 1 + (multi < B ? multi : B));
    }
    size_t o = 0;
    L.hdr = o;
    o = align256(o + 4 * (16 + 6 * (size_t)B + 4));
    L.tfr = o;
    o = align256(o + (size_t)nch * H * NTF * 512 * 2);
    L.gates = o;
    o = align256(o + (size_t)nch * H * 3 * CH * 4);
    L.slots = o;
    o = align256(o + L.nslots * (size_t)H * ((size_t)K * K + (size_t)V * K) * 4);
    L.total = o;
    return L;
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
    int VS;  // value parts (blocks per sequence, head and segment)
    int gate_dtype;
    uint32_t flags;
    float scale;
    int n_blocks;
    int cap;
    const int32_t* counts;
    const int32_t* active;
    float* capsule;
};

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: each lane names 8 bytes (four 16-bit elements) of LDS; within each group of 16
// lanes, lane i receives element i%4 of the reads of lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
}

// MFMA operands of an I/O type: bf16 I/O runs on bf16 operands (v_mfma_f32_16x16x32_bf16) and fp16
// I/O on fp16 operands (v_mfma_f32_16x16x32_f16, same rate), so the raw q, k and v rows are
// operands as they are and, with fp16 I/O, every operand keeps fp16's 11-bit significand.  pk
// rounds two fp32 values to the type (nearest even, one v_cvt_pk_*_f32); it also rounds outputs.
template <typename T>
struct Op;
template <>
struct Op<BF16> {
    using v8 = bf16x8;
    static __device__ __forceinline__ f32x4 mma(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pk(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    }
};
template <>
struct Op<F16> {
    using v8 = f16x8;
    static __device__ __forceinline__ f32x4 mma(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pk(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
    }
};
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
// sum of squares of eight 16-bit inputs, fp32: one v_dot2 per 32-bit word (the products of two
// 16-bit values are exact in fp32)
template <typename T>
__device__ __forceinline__ float sumsq8(u32x4 raw) {
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t x = raw[e];  // (a scalar first: each word is then read from its own register)
        if constexpr (std::is_same<T, F16>::value) {
            const f16x2 v = __builtin_bit_cast(f16x2, x);
            s = __builtin_amdgcn_fdot2(v, v, s, false);
        } else {
            const bf16x2 v = __builtin_bit_cast(bf16x2, x);
            s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
        }
    }
    return s;
}
// Inclusive prefix sum over the 64 lanes by DPP: shifts by 1, 2, 4 and 8 inside each 16-lane row
// (lanes past a row's start read zero), then the row totals through row_bcast:15 (row r's last lane
// into row r + 1, rows 1 and 3) and row_bcast:31 (lane 31 into rows 2 and 3).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, BOUND_ZERO));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_f32<0x111, 0xf, true>(x);   // row_shr:1
    x += dpp_f32<0x112, 0xf, true>(x);   // row_shr:2
    x += dpp_f32<0x114, 0xf, true>(x);   // row_shr:4
    x += dpp_f32<0x118, 0xf, true>(x);   // row_shr:8
    x += dpp_f32<0x142, 0xa, false>(x);  // row_bcast:15
    x += dpp_f32<0x143, 0xc, false>(x);  // row_bcast:31
    return x;
}
// e^x through the hardware 2^x (about 1 ulp): for decay factors that are rounded to bf16 or scale
// a whole chunk
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
// softplus(x) = max(x, 0) + log1p(e^-|x|) on the hardware exp2/log2, with log1p(e) = log(1 + e) e / ((1 + e) - 1)
// (the quotient cancels the rounding of 1 + e; e itself where 1 + e rounds to 1)
__device__ __forceinline__ float softplus_hw(float x) {
    const float e = fexp(-fabsf(x)), u = 1.0f + e;
    const float l1p = u == 1.0f ? e : __builtin_amdgcn_logf(u) * 0.693147180559945309f * (e / (u - 1.0f));
    return fmaxf(x, 0.0f) + l1p;
}
__device__ __forceinline__ int tf_tile(int f) { return f < 2 ? f : 2 + (f - 2) / 2; }  // token tile of T fragment f
__device__ __forceinline__ int tf_blk(int f) { return f < 2 ? 0 : (f - 2) % 2; }    // its 32-block

// Operand lane layout of v_mfma_f32_16x16x32_{bf16,f16}: lane l holds row l%16 and inner elements
// 8(l/16)..+7; the accumulator lane l holds rows 4(l/16)..+3 of column l%16.
// Plain fragment: 16 rows x 32 inner elements from `base` (row stride ld).
template <typename T>
__device__ __forceinline__ typename Op<T>::v8 frag(const uint16_t* base, int ld, int lane) {
    return *reinterpret_cast<const typename Op<T>::v8*>(base + (lane & 15) * ld + 8 * (lane >> 4));
}
// Accumulator tiles for rows 0..15 (lo) and 16..31 (hi) of a 32-row block, as one operand whose
// inner order is the split order.
template <typename T>
__device__ __forceinline__ typename Op<T>::v8 pack_acc(f32x4 lo, f32x4 hi) {
    return __builtin_bit_cast(typename Op<T>::v8, u32x4{Op<T>::pk(lo[0], lo[1]), Op<T>::pk(lo[2], lo[3]),
                                                        Op<T>::pk(hi[0], hi[1]), Op<T>::pk(hi[2], hi[3])});
}
template <typename T>
__device__ __forceinline__ u32x4 pack8(const float* x, float s) {
    return u32x4{Op<T>::pk(x[0] * s, x[1] * s), Op<T>::pk(x[2] * s, x[3] * s), Op<T>::pk(x[4] * s, x[5] * s),
                 Op<T>::pk(x[6] * s, x[7] * s)};
}
template <typename T>
__device__ __forceinline__ void unpack8(u32x4 raw, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = to_f32<T>((uint16_t)(raw[e] & 0xffffu));
        v[2 * e + 1] = to_f32<T>((uint16_t)(raw[e] >> 16));
    }
}
__device__ __forceinline__ uint16_t half_of(u32x4 w, int e) {
    return (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
}
// 4 x 4 transpose of 32-bit words across the four 16-lane rows of the wave: row r receives word r
// of rows 0..3 (out[j] = word r of row j), by two cross-half and two cross-row swaps
__device__ __forceinline__ u32x4 transpose_rows4(u32x4 x) {
    const auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return u32x4{c[0], c[1], d[0], d[1]};
}
struct Tables {
    int32_t *order, *ustart, *sstart, *slot0, *nchunk, *cstart;
};
__device__ __forceinline__ Tables tables(char* ws, int B) {
    int32_t* t = reinterpret_cast<int32_t*>(ws) + 16;
    return Tables{t, t + B, t + 2 * B + 1, t + 3 * B + 2, t + 4 * B + 3, t + 5 * B + 3};
}
__device__ __forceinline__ int nseg_of(int nch, int seglen) {
    return (seglen == INT_MAX || nch <= seglen) ? 1 : (nch + seglen - 1) / seglen;
}
// last index r in [0, n) with start[r] <= u (start[0] = 0 <= u)
__device__ __forceinline__ int find_start(const int32_t* start, int n, int u) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= u) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Exclusive scan over i < n of val(i) into out[i] (out[n] = total), by one block of 1024 threads.
template <typename F>
__device__ void block_scan(int n, F val, int32_t* out, int* s_tot, int* s_carry) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (threadIdx.x == 0) *s_carry = 0;
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
        const int i = base + (int)threadIdx.x;
        const int v = i < n ? val(i) : 0;
        int incl = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) s_tot[wv] = incl;
        __syncthreads();
        int before = *s_carry;
        for (int k = 0; k < wv; ++k) before += s_tot[k];
        if (i < n) out[i] = before + incl - v;
        __syncthreads();
        if (threadIdx.x == 1023) *s_carry = before + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) out[n] = *s_carry;
    __syncthreads();
}

// ---- index --------------------------------------------------------------------------------------
// Batches of fewer than 1024 sequences: one thread per sequence, every table formed in LDS and
// registers from a single read of the offsets (no table is read back from memory), the four scans
// in one pass.  Returns -1 (nothing done) for larger batches, else 0, or 1 for malformed offsets.
__device__ int chunk_index_small(const ChunkArgs& p) {
    const int B = p.B, i = threadIdx.x, lane = i & 63, wv = i >> 6;
    if (B >= 1024) return -1;
    __shared__ int s_off[1025], s_cnt[1024], s_part[16][4];
    int32_t* hdr = reinterpret_cast<int32_t*>(p.ws);
    int o = 0;
    if (i <= B) {
        o = p.offsets[i];
        s_off[i] = o;
    }
    __syncthreads();
    int bad = 0;
    if (i <= B) bad = (i == 0 ? o != 0 : s_off[i - 1] > o) || (i == B && o != p.N);
    const bool malformed = __syncthreads_or(bad) != 0;
    report_status(p.dev_status, malformed);
    if (malformed) {
        if (i == 0) hdr[0] = GDN_ERR_OFFSETS;
        return 1;
    }
    const Tables tb = tables(p.ws, B);
    const int sl = p.L.seglen;
    const int nc = i < B ? (s_off[i + 1] - o + CH - 1) / CH : 0;
    s_cnt[i] = nc;
    __syncthreads();
    // sequences longest first (list scheduling of the long-lived main blocks)
    int ci_rank = 0;  // chunks of the sequence of rank i
    if (i < B) {
        int rank = 0;
        for (int j = 0; j < B; ++j) {
            const int cj = s_cnt[j];
            rank += (cj > nc) || (cj == nc && j < i);
        }
        tb.order[rank] = i;
        tb.nchunk[i] = nc;
        s_off[rank] = i;  // (the offsets are no longer needed)
    }
    __syncthreads();
    if (i < B) ci_rank = s_cnt[s_off[i]];
    const int ns = nseg_of(nc, sl);
    int v[4] = {i < B ? nseg_of(ci_rank, sl) * p.H * p.VS : 0, ns > 1 ? (ns - 1) * p.H : 0, ns > 1 ? ns : 0, nc};
    int incl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        incl[e] = v[e];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl[e], d);
            if (lane >= d) incl[e] += y;
        }
        if (lane == 63) s_part[wv][e] = incl[e];
    }
    __syncthreads();
    int32_t* const outs[4] = {tb.ustart, tb.sstart, tb.slot0, tb.cstart};
    int ex[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int before = 0;
        for (int k = 0; k < wv; ++k) before += s_part[k][e];
        ex[e] = before + incl[e] - v[e];
        if (i <= B) outs[e][i] = ex[e];  // (thread B: the total)
    }
    if (i == B) {  // (the header is read only by kernels launched after this one)
        hdr[1] = ex[0];
        hdr[2] = ex[1];
        hdr[3] = ex[3];
        hdr[0] = GDN_OK;
    }
    return 0;
}

__global__ __launch_bounds__(1024) void chunk_index_kernel(ChunkArgs p) {
    if (chunk_index_small(p) >= 0) return;
    const bool malformed = offsets_malformed(p.offsets, p.B, p.N);
    report_status(p.dev_status, malformed);
    int32_t* hdr = reinterpret_cast<int32_t*>(p.ws);
    if (malformed) {
        if (threadIdx.x == 0) hdr[0] = GDN_ERR_OFFSETS;
        return;
    }
    __shared__ int s_tot[16], s_carry;
    __shared__ int s_cnt[1024];
    const Tables tb = tables(p.ws, p.B);
    const int sl = p.L.seglen;
    for (int i = threadIdx.x; i < p.B; i += blockDim.x)
        tb.nchunk[i] = (p.offsets[i + 1] - p.offsets[i] + CH - 1) / CH;
    __syncthreads();
    // sequences longest first (list scheduling of the long-lived main blocks); up to 1024 ranked
    if (p.B <= 1024) {
        const int i = threadIdx.x;
        if (i < p.B) s_cnt[i] = tb.nchunk[i];
        __syncthreads();
        if (i < p.B) {
            const int ci = s_cnt[i];
            int rank = 0;
            for (int j = 0; j < p.B; ++j) {
                const int cj = s_cnt[j];
                rank += (cj > ci) || (cj == ci && j < i);
            }
            tb.order[rank] = i;
        }
    } else {
        for (int i = threadIdx.x; i < p.B; i += blockDim.x) tb.order[i] = i;
    }
    __syncthreads();
    const int H = p.H;
    const int32_t* nchunk = tb.nchunk;
    const int32_t* order = tb.order;
    block_scan(p.B, [&](int r) { return nseg_of(nchunk[order[r]], sl) * H * p.VS; }, tb.ustart, s_tot, &s_carry);
    block_scan(p.B, [&](int i) { const int s = nseg_of(nchunk[i], sl); return s > 1 ? (s - 1) * H : 0; }, tb.sstart,
               s_tot, &s_carry);
    block_scan(p.B, [&](int i) { const int s = nseg_of(nchunk[i], sl); return s > 1 ? s : 0; }, tb.slot0, s_tot,
               &s_carry);
    block_scan(p.B, [&](int i) { return nchunk[i]; }, tb.cstart, s_tot, &s_carry);
    if (threadIdx.x == 0) {
        hdr[1] = tb.ustart[p.B];
        hdr[2] = tb.sstart[p.B];
        hdr[3] = tb.cstart[p.B];
        hdr[0] = GDN_OK;
    }
}

// ---- tmat: gates, G and the T fragments of every (chunk, head) -----------------------------------
// k rows are read whole (K/8 lanes per row, 16 bytes each); wave w normalises token rows
// 16w..16w+15 (wave 0 also forms the gates, whose loads go out first).  A is formed in its ten
// nonzero 16 x 16 blocks by MFMA, blocks w, w+4, w+8 (row-major) by wave w.  T: the four diagonal
// blocks in fp32 by forward substitution in a single wave (lane = block l/16 and column l%16, so that
// every lane does useful work; the kernel is bound by vector-ALU issue), then wave w walks down its
// block column,
// T_iw = -T_ii sum_{w <= m < i} A_im T_mw, on MFMA operands of the I/O type with its earlier blocks
// kept in accumulators (the operands of the chunk chain are rounded to that type anyway).
template <typename T, int K>
__global__ __launch_bounds__(256) void chunk_tmat_kernel(ChunkArgs p) {
    using TS = typename T::storage;
    constexpr int LPT = K / 8, TPI = 64 / LPT, NI = 16 / TPI;
    // A and T are kept as values of the operand type (a 64 x 64 tile in 9 KB each) in the space of
    // the k rows, which are dead once A's blocks are in registers: more blocks share a compute unit
    __shared__ __align__(16) union {
        uint16_t kn[CH][K + kPadRow];  // raw k rows, until A is formed
        struct {
            uint16_t am[CH][CH + 8];  // A
            uint16_t tm[CH][CH + 8];  // T
        } at;
    } r0;
    auto& am = r0.at.am;
    __shared__ __align__(16) float s_gam[CH], s_beta[CH], s_rk[CH];
    auto to16 = [](float v) { return (uint16_t)(Op<T>::pk(v, 0.0f) & 0xffffu); };

    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.ws);
    if (hdr[0] != GDN_OK) return;
    const Tables tab = tables(p.ws, p.B);
    // the H heads of a chunk on one XCD: they read the same gate rows (one cache line serves several
    // heads) and, G at a time, the same k rows
    const int blk = xcd_remap((int)blockIdx.x, p.n_blocks, p.H);
    const int cid = blk / p.H, h = blk % p.H, kh = h / p.G;
    if (cid >= hdr[3]) return;
    const int b = find_start(tab.cstart, p.B, cid);
    const int local = cid - tab.cstart[b];
    const int t0 = p.offsets[b] + local * CH;
    const int n = min(CH, p.offsets[b + 1] - t0);
    // (the wave index is read from the first lane so that the compiler keeps it, and everything
    // derived from it, in scalar registers)
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4;
    const int pc = lane % LPT, tsub = lane / LPT;
    const TS* const xk = static_cast<const TS*>(p.x.k);

    // wave 0: the raw gate inputs first, widened only after the k rows are requested too (so that
    // the three loads are in flight together)
    const bool g32 = p.gate_dtype == GDN_F32;
    uint32_t a_raw = 0u, b_raw = 0u;
    if (w == 0 && lane < n) {
        const size_t gi = (size_t)(t0 + lane) * p.H + h;
        a_raw = g32 ? static_cast<const uint32_t*>(p.a)[gi] : static_cast<const uint16_t*>(p.a)[gi];
        if (p.b) b_raw = g32 ? static_cast<const uint32_t*>(p.b)[gi] : static_cast<const uint16_t*>(p.b)[gi];
    }
    auto widen = [&](uint32_t raw) {
        return g32 ? __builtin_bit_cast(float, raw)
                   : p.gate_dtype == GDN_BF16 ? bf16_bits_to_f32((uint16_t)raw) : f16_bits_to_f32((uint16_t)raw);
    };
    u32x4 kr[NI];
    const bool kin = 8 * pc < p.K;  // keys past the width read as zero
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int ti = 16 * w + TPI * i + tsub;
        kr[i] = ti < n && kin ? *reinterpret_cast<const u32x4*>(xk + (size_t)(t0 + ti) * p.x.sk + (size_t)kh * p.K + 8 * pc)
                              : u32x4{0u, 0u, 0u, 0u};
    }
    const size_t ch = (size_t)cid * p.H + h;
    if (w == 0) {  // gates and the cumulative log-decay; padding tokens: no decay, no update
        float ell = 0.0f, beta = 0.0f;
        if (lane < n) {
            ell = -expf(p.A_log[h]) * softplus_hw(widen(a_raw) + p.dt_bias[h]);
            beta = p.b ? widen(b_raw) : 1.0f;
            if (p.b && (p.flags & GDN_SIGMOID)) beta = __builtin_amdgcn_rcpf(1.0f + fexp(-beta));
        }
        const float gam = wave_prefix_sum(ell);
        s_gam[lane] = gam;
        s_beta[lane] = beta;
        float* const gout = reinterpret_cast<float*>(p.ws + p.L.gates) + ch * 3 * CH;
        gout[lane] = gam;
        gout[CH + lane] = beta;
    }
    // raw k rows (bf16 operands); the norms 1/|k| scale A's entries instead
    float* const rkout = reinterpret_cast<float*>(p.ws + p.L.gates) + ch * 3 * CH + 2 * CH;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int ti = 16 * w + TPI * i + tsub;
        const float rk = rsqrtf(group_sum<LPT>(sumsq8<T>(kr[i])) + 1e-12f);
        *reinterpret_cast<u32x4*>(&r0.kn[ti][8 * pc]) = kr[i];
        if (pc == 0) {
            s_rk[ti] = rk;
            rkout[ti] = rk;
        }
    }
    __syncthreads();
    {  // A: lower-triangle blocks t = w, w + 4, w + 8 in row-major order (it, jt <= it), held in
       // registers until every wave is done with the k rows
        uint16_t av[3][4];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = w + NW * j;
            if (t >= 10) break;
            const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            const int jt = t - it * (it + 1) / 2;
            const int ja = 16 * jt + (lane & 15);
            const float g_ja = s_gam[ja], r_ja = s_rk[ja];
            f32x4 a = zero4();
#pragma unroll
            for (int kk = 0; kk < K; kk += 32)
                a = Op<T>::mma(frag<T>(&r0.kn[16 * it][kk], K + kPadRow, lane), frag<T>(&r0.kn[16 * jt][kk], K + kPadRow, lane), a);
            const int ia = 16 * it + 4 * g;
            const f32x4 g_ia = *reinterpret_cast<const f32x4*>(&s_gam[ia]);
            const f32x4 b_ia = *reinterpret_cast<const f32x4*>(&s_beta[ia]);
            const f32x4 r_ia = *reinterpret_cast<const f32x4*>(&s_rk[ia]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = fexp(fminf(g_ia[r] - g_ja, 0.0f));
                av[j][r] = to16((ja < ia + r) ? (b_ia[r] * r_ia[r] * r_ja) * e * a[r] : 0.0f);
            }
        }
        __syncthreads();  // k rows dead
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = w + NW * j;
            if (t >= 10) break;
            const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            const int jt = t - it * (it + 1) / 2;
#pragma unroll
            for (int r = 0; r < 4; ++r) am[16 * it + 4 * g + r][16 * jt + (lane & 15)] = av[j][r];
        }
    }
    __syncthreads();  // A ready
    auto& tm = r0.at.tm;
    if (w == (int)(blockIdx.x & 3)) {  // the four diagonal blocks by forward substitution in one wave
        const int o = 16 * g, cc = lane & 15;  // lane: block g, column l%16 of T
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == cc) ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 1; i < 16; ++i) {  // row i: x_i -= sum_{m < i} A_im x_m, the newest term last
            float a[16];
#pragma unroll
            for (int h8 = 0; h8 < (i + 7) / 8; ++h8) {
                const u32x4 r = *reinterpret_cast<const u32x4*>(&am[o + i][o + 8 * h8]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[8 * h8 + 2 * e] = to_f32<T>((uint16_t)(r[e] & 0xffffu));
                    a[8 * h8 + 2 * e + 1] = to_f32<T>((uint16_t)(r[e] >> 16));
                }
            }
#pragma unroll
            for (int m = 0; m < i; ++m) x[i] = fmaf(-a[m], x[m], x[i]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tm[o + i][o + cc] = to16(x[i]);
    }
    __syncthreads();  // diagonal blocks ready
    {  // block column w, top down: tc[m] = T_mw in accumulator layout (rows 4g..4g+3, column l%16)
        const int l16 = lane & 15;
        f32x4 tc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) tc[m][r] = m == w ? to_f32<T>(tm[16 * w + 4 * g + r][16 * w + l16]) : 0.0f;
        // A operand of rows 16 i + l%16 over the 32 columns 16 m .. 16 m + 31 in the split order
        // {4g..4g+3, 16+4g..16+4g+3}; a half whose block does not contribute is zero
        auto a_split = [&](const uint16_t* row, bool lo, bool hi) {
            const u32x2 x0 = lo ? *reinterpret_cast<const u32x2*>(row + 4 * g) : u32x2{0u, 0u};
            const u32x2 x1 = hi ? *reinterpret_cast<const u32x2*>(row + 16 + 4 * g) : u32x2{0u, 0u};
            return __builtin_bit_cast(typename Op<T>::v8, u32x4{x0[0], x0[1], x1[0], x1[1]});
        };
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            if (i <= w) continue;
            f32x4 y = zero4();
#pragma unroll
            for (int m = 0; m < 4; m += 2) {  // blocks m and m + 1 of sum_{w <= m < i} A_im T_mw
                const bool u0 = m >= w && m < i, u1 = m + 1 >= w && m + 1 < i;
                if (!u0 && !u1) continue;
                y = Op<T>::mma(a_split(&am[16 * i + l16][16 * m], u0, u1),
                               pack_acc<T>(u0 ? tc[m] : zero4(), u1 ? tc[m + 1] : zero4()), y);
            }
            const f32x4 z = Op<T>::mma(a_split(&tm[16 * i + l16][16 * i], true, false), pack_acc<T>(y, zero4()), zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) tc[i][r] = -z[r];
        }
#pragma unroll
        for (int m = 1; m < 4; ++m)
            if (m > w)
#pragma unroll
                for (int r = 0; r < 4; ++r) tm[16 * m + 4 * g + r][16 * w + l16] = to16(tc[m][r]);
    }
    __syncthreads();  // T complete
    // fragments f = w and w + 4: lane l holds row 16 it + l%16, columns 32 jj + {4g.., 16+4g..}; the
    // blocks above the diagonal are zero
    uint16_t* const tout = reinterpret_cast<uint16_t*>(p.ws + p.L.tfr) + ch * NTF * 512;
    for (int f = w; f < NTF; f += NW) {
        const int it = tf_tile(f), jj = tf_blk(f);
        const int i = 16 * it + (lane & 15);
        const int j0 = 32 * jj + 4 * g, j1 = j0 + 16;
        const u32x2 x0 = (j0 >> 4) <= it ? *reinterpret_cast<const u32x2*>(&tm[i][j0]) : u32x2{0u, 0u};
        const u32x2 x1 = (j1 >> 4) <= it ? *reinterpret_cast<const u32x2*>(&tm[i][j1]) : u32x2{0u, 0u};
        *reinterpret_cast<u32x4*>(tout + f * 512 + 8 * lane) = u32x4{x0[0], x0[1], x1[0], x1[1]};
    }
}

// ---- summary and main -----------------------------------------------------------------------------
// LDS layouts of one chunk (all 16-bit elements):
//   kn, qn  [token][key]: the raw k and q rows as operands (the L2 norms 1/|k|, 1/|q| scale
//           per-token factors instead), keys of every 32-block in the split order (physical slot
//           8g + e holds key 4g + e for e < 4 and 16 + 4g + e - 4 otherwise), so a split fragment
//           is one 16-byte read; products between two such rows are unchanged.  Four consecutive
//           keys share 8 contiguous bytes, which is what the transposing read of K^T takes.
//   vr      [token][value column]: the v rows as loaded.
//   kt      [key][token] (fp16 operands): transposed, tokens of every 32-block in the split order,
//           in 16-byte units (8 tokens = one lane group's split fragment) placed at unit u ^ (idx/8 % 8)
//           so that the stores of one row-major lane (8 consecutive indices) spread over the banks.
//   pb      P, [row i][column j] with the columns in the split order.
__device__ __forceinline__ int split_key_slot(int pc) {  // slot of keys 8pc..8pc+3 (then +8 for 8pc+4..+7)
    const int a = pc & 3;
    return 32 * (pc >> 2) + 16 * (a & 1) + 4 * (a >> 1);
}
#ifndef GDN_TSWZ
#define GDN_TSWZ 4
#endif
constexpr int kSwz = GDN_TSWZ;
// element offset of token t in row idx of a transposed tile
__device__ __forceinline__ int tpos(int idx, int t) {
    const int q = (t >> 2) & 7;
    const int unit = 4 * (t >> 5) + (q & 3);
    return 8 * (unit ^ ((idx >> kSwz) & 7)) + 4 * (q >> 2) + (t & 3);
}
// split fragment of a transposed tile: rows idx0 + l%16, the tokens of 32-block jj
template <typename T>
__device__ __forceinline__ typename Op<T>::v8 frag_t(const uint16_t* tile, int ld, int idx0, int jj, int lane) {
    const int idx = idx0 + (lane & 15);
    return *reinterpret_cast<const typename Op<T>::v8*>(tile + idx * ld + 8 * ((4 * jj + (lane >> 4)) ^ ((idx >> kSwz) & 7)));
}

// qn and vr are last read before a chunk's middle barrier and are written for the next chunk after
// it, so one copy serves; the per-token factors are read after that barrier and have two, and so has
// the source of K^T (kn on bf16 operands, kt on fp16 ones) where LDS allows (else the next chunk's
// copy waits for one more barrier).
struct ChunkBuf {
    // per token: G; b; scale e^G; b e^G / |k|; e^{G_C - G} / |k|; 1/|k|; 1/|q|; and e^{G_C}
    float gam[CH], beta[CH], eg[CH], bx[CH], ud[CH], rk[CH], rq[CH], gc[4];
};
// TRK (bf16 operands): K^T is read from the k rows themselves through the transposing read, so the k
// rows take NKT copies and there is no transposed tile; on fp16 operands K^T holds the normalised
// rows and has a tile of its own (NKT copies).
template <int K, int VT, bool SUMMARY, int NKT, bool SO, bool TRK>
struct FusedLds {
    uint16_t kn[TRK ? NKT : 1][CH][K + kPadRow];
    uint16_t qn[SUMMARY ? 1 : CH][K + kPadRow];
    uint16_t vr[CH][VT + kPadRow];  // v rows as loaded (read transposed by ds_read_b64_tr_b16)
    uint16_t tf[NTF][512];  // T fragments (lane order), read before the middle barrier
    uint16_t kt[TRK ? 1 : NKT][TRK ? 1 : K][CH + kPadT];
    ChunkBuf buf[2];
    uint16_t pb[SUMMARY ? 1 : CH][CH + kPadT];
    uint16_t ob[SUMMARY || !SO ? 1 : CH][VT + 8];  // output rows of the previous chunk, stored whole
};
// LDS of one block: two copies of the K^T source and staged output rows while they fit, else one
// copy, and then output rows stored straight from the registers (K = 256 with 128-column value
// parts on fp16 operands).
constexpr size_t kLdsBytes = 160 * 1024;
template <int K, int VT, bool SUMMARY, bool TRK>
struct LdsPlan {
    static constexpr int NKT = sizeof(FusedLds<K, VT, SUMMARY, 2, true, TRK>) <= kLdsBytes ? 2 : 1;
    static constexpr bool SO = sizeof(FusedLds<K, VT, SUMMARY, NKT, true, TRK>) <= kLdsBytes;
    using Lds = FusedLds<K, VT, SUMMARY, NKT, SO, TRK>;
    static_assert(sizeof(Lds) <= kLdsBytes, "LDS per block");
};
// voffset of a buffer access that is to read zero or write nothing (past every range used here:
// the ranges stay below 2^30 bytes)
constexpr int kOutOfRange = 0x7ff00000;

// MODE: kMain, kMainCapture (also records the first tokens of each sequence) or kSummary.
constexpr int kMain = 0, kMainCapture = 1, kSummary = 2;

// One block per (segment, head, value part) of VT columns; one wave per VTW 16-column value tiles.
// K is the compiled key width (p.K the real one), VT the part's width (p.V the real value width).
// Staging: wave w stages token rows RPW w .. RPW w + RPW-1.
template <typename T, int K, int VT, int MODE, int VTW>
__global__ __launch_bounds__(64 * (VT / (16 * VTW))) void chunk_fused_kernel(ChunkArgs p) {
    using TS = typename T::storage;
    using OpV = typename Op<T>::v8;
    constexpr bool SUMMARY = MODE == kSummary, CAPTURE = MODE == kMainCapture;
    constexpr int NWV = VT / (16 * VTW);  // waves
    static_assert(K % 32 == 0 && VT % (16 * VTW) == 0 && (!SUMMARY || K % (16 * NWV) == 0), "tile shapes");
    constexpr int NPHI = SUMMARY ? K / (16 * NWV) : 0;  // Phi column tiles per wave in a summary
    constexpr int NCT = VTW + NPHI;
    constexpr int KT = K / 16, KK = K / 32;
    constexpr int RPW = CH / NWV;  // token rows staged per wave
    constexpr int LPT = K / 8, TPI = 64 / LPT;  // k/q rows: lanes per row, rows per instruction
    constexpr int LPV = VT / 8, TPV = 64 / LPV;
    static_assert(RPW % TPI == 0 && RPW % TPV == 0, "staging tiles");
    constexpr int NI = RPW / TPI, NV = RPW / TPV;
    constexpr bool TRK = std::is_same<T, BF16>::value;
    using Plan = LdsPlan<K, VT, SUMMARY, TRK>;
    constexpr int NKT = Plan::NKT;
    constexpr bool SO = Plan::SO;
    __shared__ __align__(16) typename Plan::Lds sm;

    int32_t* hdr = reinterpret_cast<int32_t*>(p.ws);
    if (hdr[0] != GDN_OK) return;
    const Tables tab = tables(p.ws, p.B);
    const int u = xcd_remap((int)blockIdx.x, p.n_blocks, p.G * p.VS);
    if (u >= hdr[SUMMARY ? 2 : 1]) return;
    int b, local;
    if constexpr (SUMMARY) {
        b = find_start(tab.sstart, p.B, u);
        local = u - tab.sstart[b];
    } else {
        const int r = find_start(tab.ustart, p.B, u);
        b = tab.order[r];
        local = u - tab.ustart[r];
    }
    // the value parts of a head, then the heads of a key-head group, are adjacent units (they read
    // the same k and q rows)
    const int HV = p.H * p.VS;
    const int seg = local / HV, h = (local % HV) / p.VS, vp = local % p.VS, kh = h / p.G;
    const int Kr = p.K, Vr = p.V, v0 = VT * vp;  // real widths; first value column of this block
    const int sl = p.L.seglen;
    const int nch = tab.nchunk[b];
    const int nseg = nseg_of(nch, sl);
    const int cb = nseg == 1 ? 0 : seg * sl;
    const int ce = nseg == 1 ? nch : min(nch, cb + sl);
    const int seq_start = p.offsets[b], len = p.offsets[b + 1] - seq_start;
    const int cid0 = tab.cstart[b];

    // (the wave index is read from the first lane so that the compiler keeps it, and everything
    // derived from it, in scalar registers: wave-dependent buffer resources, loop bounds)
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4,
              l16 = lane & 15;
    const size_t slot_stride = ((size_t)K * K + (size_t)VT * K);
    float* const slots = reinterpret_cast<float*>(p.ws + p.L.slots);
    auto slot_phi = [&](int s) { return slots + ((size_t)s * p.H + h) * slot_stride; };
    auto slot_n = [&](int s) { return slot_phi(s) + (size_t)K * K; };

    // column of tile ct of this lane within the part: value column 16 (VTW w + ct) + l%16 (ct < VTW),
    // or (summary) Phi column 16 (NPHI w + ct - VTW) + l%16
    auto col_of = [&](int ct) {
        return ct < VTW ? 16 * (VTW * w + ct) + l16 : VT + 16 * (NPHI * w + ct - VTW) + l16;
    };

    // ---- entering state: sacc[kt][ct] = S0^T[16 kt + 4g .. +3][col]; a state tensor has the real
    // widths (keys and columns past them are zero here), a slot the compiled ones
    f32x4 sacc[KT][NCT];
    {
        const float* src = nullptr;
        bool from_slot = false;
        if constexpr (!SUMMARY) {
            if (nseg == 1) {
                src = p.state_in ? p.state_in + ((size_t)b * p.H + h) * Vr * Kr : nullptr;
            } else {
                src = slot_n(tab.slot0[b] + (seg == 0 ? nseg - 1 : seg - 1));
                from_slot = true;
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = col_of(ct);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int k0 = 16 * kt + 4 * g;
                if (ct < VTW) {
                    if (from_slot) sacc[kt][ct] = *reinterpret_cast<const f32x4*>(src + (size_t)c * K + k0);
                    else if (src && v0 + c < Vr && k0 < Kr)
                        sacc[kt][ct] = *reinterpret_cast<const f32x4*>(src + (size_t)(v0 + c) * Kr + k0);
                    else sacc[kt][ct] = zero4();
                } else {  // Phi starts as the identity
                    const int cc = c - VT;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[kt][ct][r] = (k0 + r == cc) ? 1.0f : 0.0f;
                }
            }
        }
    }

    // ---- capture (first segment): zero the unrecorded slots (the first value part); g and k^ are
    // recorded by the first value part, delta by each part for its columns
    int captured = 0;
    CaptureRow crow{};
    if constexpr (CAPTURE) {
        if (seg == 0) {
            captured = captured_tokens(p.counts, p.active, p.cap, b, len);
            crow = capture_row(p.capsule, b, p.cap, p.H, p.HQ, Kr, Vr);
            if (vp == 0) {
                for (int i = captured; i < p.cap; ++i) {
                    if (tid == 0) *crow.g(i, h) = 0.0f;
                    for (int j = tid; j < Vr; j += blockDim.x) crow.d(i, h)[j] = 0.0f;
                    if (h % p.G == 0)
                        for (int j = tid; j < Kr; j += blockDim.x) crow.k(i, kh)[j] = 0.0f;
                }
            }
        }
    }

    const TS* const xq = static_cast<const TS*>(p.x.q);
    const TS* const xk = static_cast<const TS*>(p.x.k);
    const TS* const xv = static_cast<const TS*>(p.x.v);
    const uint16_t* const tfr = reinterpret_cast<const uint16_t*>(p.ws + p.L.tfr);
    const float* const gts = reinterpret_cast<const float*>(p.ws + p.L.gates);
    const int pc = lane % LPT, tsub = lane / LPT;
    const int pv = lane % LPV, vsub = lane / LPV;
    const int ks0 = split_key_slot(pc);
    constexpr int RSRC = 0x00020000;  // raw buffer resource (gfx9 family)
    // this lane's 8 keys of a k/q row and 8 columns of a v/output row exist (else zero / not written)
    const bool kin = 8 * pc < Kr, vin = v0 + 8 * pv < Vr;

    // Rows of one chunk (range-checked buffer loads: rows at or past the chunk's end read as zero),
    // T fragments w, w + NWV, .. (one copy per block; fragments past the last read as zero) and, in
    // wave 0 only, the tokens' G, b and 1/|k| (lane = token; the other waves' range is empty).
    constexpr int NTFW = (NTF + NWV - 1) / NWV;
    struct Rows {
        u32x4 k[NI], q[SUMMARY ? 1 : NI], v[NV];
        u32x4 tf[NTFW];
        float gam, beta, rk;
    };
    auto load_rows = [&](int c, Rows& R) {
        const int t0 = seq_start + c * CH, n = min(CH, len - c * CH);
        const size_t ch = (size_t)(cid0 + c) * p.H + h;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<TS*>(xk + (size_t)t0 * p.x.sk + (size_t)kh * Kr), 0, n * (int)p.x.sk * (int)sizeof(TS), RSRC);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<TS*>(xv + (size_t)t0 * p.x.sv + (size_t)h * Vr + v0), 0, n * (int)p.x.sv * (int)sizeof(TS), RSRC);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int ti = RPW * w + TPI * i + tsub;
            R.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rk, kin ? (ti * (int)p.x.sk + 8 * pc) * (int)sizeof(TS) : kOutOfRange, 0, 0));
        }
        if constexpr (!SUMMARY) {
            const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<TS*>(xq + (size_t)t0 * p.x.sq + (size_t)kh * Kr), 0, n * (int)p.x.sq * (int)sizeof(TS), RSRC);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int ti = RPW * w + TPI * i + tsub;
                R.q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rq, kin ? (ti * (int)p.x.sq + 8 * pc) * (int)sizeof(TS) : kOutOfRange, 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int ti = RPW * w + TPV * i + vsub;
            R.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rv, vin ? (ti * (int)p.x.sv + 8 * pv) * (int)sizeof(TS) : kOutOfRange, 0, 0));
        }
        const __amdgpu_buffer_rsrc_t rt =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(tfr + ch * NTF * 512), 0, NTF * 1024, RSRC);
#pragma unroll
        for (int j = 0; j < NTFW; ++j)
            R.tf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rt, ((w + NWV * j) * 512 + 8 * lane) * 2, 0, 0));
        const __amdgpu_buffer_rsrc_t rgt =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(gts + ch * 3 * CH), 0, w == 0 ? 3 * CH * 4 : 0, RSRC);
        R.gam = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgt, lane * 4, 0, 0));
        R.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgt, (CH + lane) * 4, 0, 0));
        R.rk = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgt, (2 * CH + lane) * 4, 0, 0));
    };
    // raw rows, transposes, norms and per-token factors of chunk c into buffer Bf
    // K^T operand from the row-major k rows (bf16 operands): keys 16 kt + l%16, the tokens of 32-block
    // jj in the split order.  Within each 16-lane group g, lane s names 8 bytes of token
    // 32 jj + 4g + s/4 (then 16 tokens on) at the split slots of keys 16 kt + 4(s%4) .. +3; the
    // transposing read hands each key's four tokens to that key's lane.
    auto kt_frag = [&](const uint16_t (&kr)[CH][K + kPadRow], int kt, int jj) -> OpV {
        const int col = 32 * (kt >> 1) + 8 * (l16 & 3) + 4 * (kt & 1);
        const v4i16 lo = lds_read_tr16(&kr[32 * jj + 4 * g + (l16 >> 2)][col]);
        const v4i16 hi = lds_read_tr16(&kr[32 * jj + 16 + 4 * g + (l16 >> 2)][col]);
        return __builtin_bit_cast(OpV, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto stage = [&](int c, const Rows& R, ChunkBuf& Bf, int kbuf) {
        auto& knb = sm.kn[TRK ? kbuf : 0];
        auto& kt = sm.kt[TRK ? 0 : kbuf];
        const bool cap_chunk = CAPTURE && c == 0 && captured > 0;
#pragma unroll
        for (int j = 0; j < NTFW; ++j)
            if (w + NWV * j < NTF) *reinterpret_cast<u32x4*>(&sm.tf[w + NWV * j][8 * lane]) = R.tf[j];
        if (w == 0) {  // (every value part: each reads its own factors)
            const float gC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, R.gam), CH - 1));
            const float eg = fexp(R.gam);
            Bf.gam[lane] = R.gam;
            Bf.beta[lane] = R.beta;
            Bf.eg[lane] = p.scale * eg;
            Bf.bx[lane] = R.beta * eg * R.rk;
            Bf.ud[lane] = std::is_same<T, F16>::value ? fexp(gC - R.gam) : fexp(gC - R.gam) * R.rk;
            Bf.rk[lane] = R.rk;
            if (lane == 0) Bf.gc[0] = fexp(gC);
            // the previous token's G, read by the whole wave (a lane shuffle from an inactive lane
            // would read zero)
            const float gprev = __shfl(R.gam, (lane + CH - 1) & (CH - 1));
            if (cap_chunk && vp == 0 && lane < captured) *crow.g(lane, h) = expf(R.gam - (lane > 0 ? gprev : 0.0f));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int ti = RPW * w + TPI * i + tsub;
            const u32x4 kb = R.k[i];
            *reinterpret_cast<u32x2*>(&knb[ti][ks0]) = u32x2{kb[0], kb[1]};
            *reinterpret_cast<u32x2*>(&knb[ti][ks0 + 8]) = u32x2{kb[2], kb[3]};
            // K^T: raw rows on bf16 operands (1/|k| goes with U), read from the k rows; on fp16
            // operands the rows are normalised here, so that U's factor stays within 1 whatever |k|
            // is, and transposed into a tile of their own
            if constexpr (!TRK) {
                u32x4 ktb = kb;
                if constexpr (std::is_same<T, F16>::value) {
                    const float rk = rsqrtf(group_sum<LPT>(sumsq8<T>(kb)) + 1e-12f);
                    float kf[8];
                    unpack8<T>(kb, kf);
                    ktb = pack8<T>(kf, rk);
                }
                if constexpr (TPI == 4) {
                    // lanes pc, pc + 16, pc + 32, pc + 48 hold four consecutive tokens: after the
                    // transpose, row tsub has keys 8 pc + 2 tsub and + 1 of all four (8 bytes per key)
                    const u32x4 y = transpose_rows4(ktb);
                    const int r0 = 8 * pc + 2 * tsub, t0 = RPW * w + TPI * i;
                    *reinterpret_cast<u32x2*>(&kt[r0][tpos(r0, t0)]) =
                        u32x2{(y[0] & 0xffffu) | (y[1] << 16), (y[2] & 0xffffu) | (y[3] << 16)};
                    *reinterpret_cast<u32x2*>(&kt[r0 + 1][tpos(r0 + 1, t0)]) =
                        u32x2{(y[0] >> 16) | (y[1] & 0xffff0000u), (y[2] >> 16) | (y[3] & 0xffff0000u)};
                } else {
                    const int tp = tpos(8 * pc, ti);
    #pragma unroll
                    for (int e = 0; e < 8; ++e) kt[8 * pc + e][tp] = half_of(ktb, e);
                }
            }
            if constexpr (!SUMMARY) {
                if (cap_chunk && ti < captured && h % p.G == 0 && vp == 0) {  // (uniform over the row's lanes)
                    const float rk = rsqrtf(group_sum<LPT>(sumsq8<T>(R.k[i])) + 1e-12f);
                    float kf[8];
                    unpack8<T>(R.k[i], kf);
                    if (kin)
#pragma unroll
                        for (int e = 0; e < 8; ++e) crow.k(ti, kh)[8 * pc + e] = kf[e] * rk;
                }
                const u32x4 qb = R.q[i];
                *reinterpret_cast<u32x2*>(&sm.qn[ti][ks0]) = u32x2{qb[0], qb[1]};
                *reinterpret_cast<u32x2*>(&sm.qn[ti][ks0 + 8]) = u32x2{qb[2], qb[3]};
                const float rq = rsqrtf(group_sum<LPT>(sumsq8<T>(R.q[i])) + 1e-12f);
                if (pc == 0) Bf.rq[ti] = rq;
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {  // v rows as loaded: 16 bytes a lane
            const int ti = RPW * w + TPV * i + vsub;
            *reinterpret_cast<u32x4*>(&sm.vr[ti][8 * pv]) = R.v[i];
        }
    };

    if constexpr (!SUMMARY) {  // P blocks (0,1) and (2,3) are read as zeros by the U^T P^T products
        for (int z = tid; z < 128; z += blockDim.x) {
            const int blk2 = z >> 6, rr = (z & 63) >> 2, cc = z & 3;
            *reinterpret_cast<u32x2*>(&sm.pb[32 * blk2 + rr][32 * blk2 + 8 * cc + 4]) = u32x2{0u, 0u};
        }
    }
    TS* const outp = static_cast<TS*>(p.out);
    // Output rows of chunk c (written to LDS by its O step, read after the next barrier): wave w
    // stores token rows RPW w .. + RPW-1 whole, 16 bytes a lane; rows at or past the chunk's end
    // are dropped by the range-checked buffer (so every store is issued and the waits stay exact)
    auto flush_out = [&](int c) {
        if constexpr (!SUMMARY && SO) {
            const int t0 = seq_start + c * CH, n = min(CH, len - c * CH);
            const __amdgpu_buffer_rsrc_t orsrc =
                __builtin_amdgcn_make_buffer_rsrc(outp + (size_t)t0 * p.H * Vr, 0, n * p.H * Vr * (int)sizeof(TS), RSRC);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int ti = RPW * w + TPV * i + vsub;
                const u32x4 val = *reinterpret_cast<const u32x4*>(&sm.ob[ti][8 * pv]);
                __builtin_amdgcn_raw_buffer_store_b128(
                    val, orsrc, vin ? ((ti * p.H + h) * Vr + v0 + 8 * pv) * (int)sizeof(TS) : kOutOfRange, 0, 0);
            }
        }
    };

    // One chunk; Bf and K^T buffer kc hold it, Bn and buffer kx receive the next one (the buffers
    // alternate; with one K^T buffer kc and kx are the same)
    Rows R;
    auto step = [&](int c, ChunkBuf& Bf, ChunkBuf& Bn, int kc, int kx) {
        const auto& knc = sm.kn[TRK ? kc : 0];
        const int t0 = seq_start + c * CH, n = min(CH, len - c * CH);
        const bool cap_chunk = CAPTURE && c == 0 && captured > 0;
        if (c > cb) flush_out(c - 1);
        if (c + 1 < ce) load_rows(c + 1, R);  // in flight during this chunk

        // ---- P = M o (Q K^T) / (|q_i| |k_j|): the ten nonzero 16 x 16 blocks (it, jt <= it), formed
        // transposed (K_jt Q_it^T; lane: 4 consecutive j = 16 jt + 4g + r of row i = 16 it + l%16).
        // Block n goes to wave (n + 2) % NWV: the waves with a second block then sit on other SIMDs
        // than wave 0, which also forms the per-token factors (waves w and w + 4 share a SIMD).
        if constexpr (!SUMMARY) {
#pragma unroll
            for (int nb = (w + NWV - 2 % NWV) % NWV; nb < 10; nb += NWV) {
                const int it = nb < 1 ? 0 : nb < 3 ? 1 : nb < 6 ? 2 : 3;
                const int jt = nb - it * (it + 1) / 2;
                f32x4 pt = zero4();
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    pt = Op<T>::mma(frag<T>(&knc[16 * jt][32 * kk], K + kPadRow, lane), frag<T>(&sm.qn[16 * it][32 * kk], K + kPadRow, lane), pt);
                const int i = 16 * it + l16, j0 = 16 * jt + 4 * g;
                const float g_i = Bf.gam[i], q_i = Bf.rq[i];
                const f32x4 g_j = *reinterpret_cast<const f32x4*>(&Bf.gam[j0]);
                const f32x4 r_j = *reinterpret_cast<const f32x4*>(&Bf.rk[j0]);
                float pv4[4];
                if (it == jt) {  // diagonal block: the causal mask (every lane computes a finite value
                                 // and the mask selects it: no divergent branch)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float val = fexp(fminf(g_i - g_j[r], 0.0f)) * (q_i * r_j[r]) * pt[r];
                        pv4[r] = j0 + r <= i ? val : 0.0f;
                    }
                } else {  // below the diagonal: j < i, and G does not increase along the chunk
#pragma unroll
                    for (int r = 0; r < 4; ++r) pv4[r] = fexp(g_i - g_j[r]) * (q_i * r_j[r]) * pt[r];
                }
                *reinterpret_cast<u32x2*>(&sm.pb[i][32 * (jt >> 1) + 8 * g + 4 * (jt & 1)]) =
                    u32x2{Op<T>::pk(pv4[0], pv4[1]), Op<T>::pk(pv4[2], pv4[3])};
            }
        }

        // ---- chain: S0^T -> K S0^T (and S0 Q^T) -> R -> U -> S
        OpV sbf[KK][NCT];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) sbf[kk][ct] = pack_acc<T>(sacc[2 * kk][ct], sacc[2 * kk + 1][ct]);
        f32x4 ks[4][NCT];
        f32x4 oq[SUMMARY ? 1 : 4][VTW];  // (S0 Q^T) tiles: rows = value columns, columns = tokens
#pragma unroll
        for (int it = 0; it < 4; ++it) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) ks[it][ct] = zero4();
            if constexpr (!SUMMARY) {
#pragma unroll
                for (int ct = 0; ct < VTW; ++ct) oq[it][ct] = zero4();
            }
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const OpV kf = frag<T>(&knc[16 * it][32 * kk], K + kPadRow, lane);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ks[it][ct] = Op<T>::mma(kf, sbf[kk][ct], ks[it][ct]);
                if constexpr (!SUMMARY) {
                    const OpV qf = frag<T>(&sm.qn[16 * it][32 * kk], K + kPadRow, lane);
#pragma unroll
                    for (int ct = 0; ct < VTW; ++ct) oq[it][ct] = Op<T>::mma(sbf[kk][ct], qf, oq[it][ct]);
                }
            }
        }
        // R = diag(b) V - diag(b e^G / |k|) (K S0^T), in place of ks (rows 16 it + 4g + r)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i0 = 16 * it + 4 * g;
            const f32x4 bet = *reinterpret_cast<const f32x4*>(&Bf.beta[i0]);
            const f32x4 bxv = *reinterpret_cast<const f32x4*>(&Bf.bx[i0]);
#pragma unroll
            for (int ct = 0; ct < VTW; ++ct) {
                // tokens i0 .. i0+3 of column 16 (VTW w + ct) + l%16 from the row-major v tile: within
                // each 16-lane group the transposing read hands lane i element i%4 of the four lanes
                // 4k + i/4 (k = 0..3), so lane s reads token i0 + s/4, columns + 4 (s%4) .. + 3
                const v4i16 tv = lds_read_tr16(&sm.vr[i0 + (l16 >> 2)][16 * (VTW * w + ct) + 4 * (l16 & 3)]);
                const float vv[4] = {to_f32<T>((uint16_t)tv[0]), to_f32<T>((uint16_t)tv[1]), to_f32<T>((uint16_t)tv[2]),
                                     to_f32<T>((uint16_t)tv[3])};
#pragma unroll
                for (int r = 0; r < 4; ++r) ks[it][ct][r] = fmaf(bet[r], vv[r], -bxv[r] * ks[it][ct][r]);
            }
#pragma unroll
            for (int ct = VTW; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) ks[it][ct][r] = -bxv[r] * ks[it][ct][r];
        }
        // U = T R (T lower triangular: token tiles 0 and 1 need only the first 32-block)
        f32x4 ua[4][NCT];
        {
            OpV tf[NTF];
#pragma unroll
            for (int f = 0; f < NTF; ++f) tf[f] = *reinterpret_cast<const OpV*>(&sm.tf[f][8 * lane]);
            OpV rb[2][NCT];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) rb[jj][ct] = pack_acc<T>(ks[2 * jj][ct], ks[2 * jj + 1][ct]);
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ua[it][ct] = zero4();
#pragma unroll
            for (int f = 0; f < NTF; ++f) {
                const int it = tf_tile(f), jj = tf_blk(f);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ua[it][ct] = Op<T>::mma(tf[f], rb[jj][ct], ua[it][ct]);
            }
        }
        // P is complete, and qn, vr and (on fp16 operands) kn of this chunk have been read for the
        // last time (the next chunk's rows are staged into them after the state update)
        __syncthreads();
        if constexpr (!SUMMARY) {
            // O^T = (S0 Q^T) diag(scale e^G / |q|) + scale U^T P^T (the first factor is eg / |q|).
            // Lane: value columns 16 w + 4g .. +3 of token 16 it + l%16, into the LDS output rows
            OpV ub[2][VTW];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int ct = 0; ct < VTW; ++ct) ub[jj][ct] = pack_acc<T>(ua[2 * jj][ct], ua[2 * jj + 1][ct]);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int i = 16 * it + l16;
                const OpV p0 = frag<T>(&sm.pb[16 * it][0], CH + kPadT, lane);
                OpV p1;
                if (it >= 2) p1 = frag<T>(&sm.pb[16 * it][32], CH + kPadT, lane);
                const float qf = Bf.eg[i] * Bf.rq[i];
#pragma unroll
                for (int ct = 0; ct < VTW; ++ct) {
                    f32x4 o = Op<T>::mma(ub[0][ct], p0, zero4());
                    if (it >= 2) o = Op<T>::mma(ub[1][ct], p1, o);
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = fmaf(oq[it][ct][r], qf, p.scale * o[r]);
                    const u32x2 ov = u32x2{Op<T>::pk(o[0], o[1]), Op<T>::pk(o[2], o[3])};
                    const int oc = 16 * (VTW * w + ct) + 4 * g;
                    if constexpr (SO) {
                        *reinterpret_cast<u32x2*>(&sm.ob[16 * it + l16][oc]) = ov;
                    } else if (i < n && v0 + oc < Vr) {
                        *reinterpret_cast<u32x2*>(outp + ((size_t)(t0 + i) * p.H + h) * Vr + v0 + oc) = ov;
                    }
                }
            }
            if (cap_chunk) {  // delta of the recorded tokens (at most one chunk): rows of U
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int ct = 0; ct < VTW; ++ct)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (16 * it + 4 * g + r < captured && v0 + col_of(ct) < Vr)
                                crow.d(16 * it + 4 * g + r, h)[v0 + col_of(ct)] = ua[it][ct][r];
            }
        }
        // S0^T <- e^{G_C} S0^T + K^T diag(e^{G_C - G} / |k|) U
        {
            OpV udb[2][NCT];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(&Bf.ud[32 * jj + 4 * g]);
                const f32x4 d1 = *reinterpret_cast<const f32x4*>(&Bf.ud[32 * jj + 16 + 4 * g]);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) udb[jj][ct] = pack_acc<T>(ua[2 * jj][ct] * d0, ua[2 * jj + 1][ct] * d1);
            }
            const float gC = Bf.gc[0];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const OpV a0 = TRK ? kt_frag(knc, kt, 0) : frag_t<T>(&sm.kt[kc][0][0], CH + kPadT, 16 * kt, 0, lane);
                const OpV a1 = TRK ? kt_frag(knc, kt, 1) : frag_t<T>(&sm.kt[kc][0][0], CH + kPadT, 16 * kt, 1, lane);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 s = sacc[kt][ct] * gC;
                    s = Op<T>::mma(a0, udb[0][ct], s);
                    sacc[kt][ct] = Op<T>::mma(a1, udb[1][ct], s);
                }
            }
        }
        // the next chunk into the other buffer (last read before the previous barrier); a single kt
        // buffer is free once every wave has updated its state
        if constexpr (NKT == 1) __syncthreads();
        if (c + 1 < ce) stage(c + 1, R, Bn, kx);
        __syncthreads();
    };

    if (cb < ce) {
        load_rows(cb, R);
        stage(cb, R, sm.buf[0], 0);
    }
    // nothing may be in flight when the loop starts: the compiler then has to wait in the loop only
    // for what the loop itself issued
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int c = cb; c < ce; ++c) {
        const int bi = (c - cb) & 1;
        step(c, sm.buf[bi], sm.buf[bi ^ 1], NKT == 2 ? bi : 0, NKT == 2 ? bi ^ 1 : 0);
    }
    if (cb < ce) flush_out(ce - 1);  // after the last step's barrier

    // ---- leaving state
    if constexpr (SUMMARY) {
        float* const phi = slot_phi(tab.slot0[b] + seg);
        float* const nst = slot_n(tab.slot0[b] + seg);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int c = col_of(ct);
            float* dst = ct < VTW ? nst + (size_t)c * K : phi + (size_t)(c - VT) * K;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) *reinterpret_cast<f32x4*>(dst + 16 * kt + 4 * g) = sacc[kt][ct];
        }
    } else {
        if (seg == nseg - 1 && p.state_out != nullptr) {
            float* const dst = p.state_out + ((size_t)b * p.H + h) * Vr * Kr;
#pragma unroll
            for (int ct = 0; ct < VTW; ++ct) {
                const int c = v0 + col_of(ct);
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
                    if (c < Vr && 16 * kt + 4 * g < Kr)
                        *reinterpret_cast<f32x4*>(dst + (size_t)c * Kr + 16 * kt + 4 * g) = sacc[kt][ct];
            }
        }
    }
}

// ---- combine: S_start of every segment, in order ------------------------------------------------
// K and V are the compiled widths (the slots' layout; one value part).
// One block per (sequence, head, 8 value rows); a thread owns key column k = t % K of rows
// t / K + (NTH / K) j.  S_start(s+1) = S_start(s) Phi_s + N_s  (rows v: S[v][k] = sum_c S[v][c]
// phi[c][k] + N[v][k]), in fp32.  Phi is staged through LDS in tiles of CT rows; the next tile (and
// the next N rows) are loaded into registers while the current one is used.
// NTH = 256 threads (more threads per block with fewer rows each measured slower).
template <int K>
constexpr int combine_threads() { return 256; }
template <int K, int V>
__global__ __launch_bounds__(combine_threads<K>()) void chunk_combine_kernel(ChunkArgs p) {
    constexpr int NTH = combine_threads<K>();
    constexpr int VR = 8;          // value rows per block
    constexpr int RG = NTH / K;    // row groups
    constexpr int RPT = VR / RG;   // rows per thread
    constexpr int CT = K * K <= 16384 ? K : 16384 / K;  // Phi rows per tile
    constexpr int NCT = K / CT;
    constexpr int NLD = CT * K / (4 * NTH);  // 16-byte loads per thread per tile
    static_assert(NTH % K == 0 && VR % RG == 0 && NLD >= 1 && V % VR == 0, "combine tiling");
    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.ws);
    if (hdr[0] != GDN_OK) return;
    const Tables tab = tables(p.ws, p.B);
    constexpr int NVT = V / VR;
    // the NVT blocks of a (sequence, head) on one XCD: each reads every Phi of the head, which its
    // L2 then serves once
    const int blk = xcd_remap((int)blockIdx.x, (int)gridDim.x, NVT);
    const int vt = blk % NVT, bh = blk / NVT;
    const int h = bh % p.H, b = bh / p.H;
    const int nseg = nseg_of(tab.nchunk[b], p.L.seglen);
    if (nseg <= 1) return;
    __shared__ __align__(16) float phs[CT * K];
    __shared__ __align__(16) float s[VR][K];
    const int tid = threadIdx.x, k = tid % K, rg = tid / K;
    const size_t slot_stride = ((size_t)K * K + (size_t)V * K);
    float* const slots = reinterpret_cast<float*>(p.ws + p.L.slots);
    auto slot_phi = [&](int sidx) { return slots + ((size_t)sidx * p.H + h) * slot_stride; };
    const int s0 = tab.slot0[b];
    float acc[RPT];
    {
        float* const st0 = slot_phi(s0 + nseg - 1) + (size_t)K * K;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int v = VR * vt + rg + RG * j;
            acc[j] = p.state_in && v < p.V && k < p.K ? p.state_in[(((size_t)b * p.H + h) * p.V + v) * p.K + k] : 0.0f;
            s[rg + RG * j][k] = acc[j];
            st0[(size_t)v * K + k] = acc[j];
        }
    }
    f32x4 pre[NLD];
    float npre[RPT];
    auto fetch = [&](int sg, int ct) {
        const f32x4* src = reinterpret_cast<const f32x4*>(slot_phi(s0 + sg) + (size_t)ct * CT * K);
#pragma unroll
        for (int i = 0; i < NLD; ++i) pre[i] = src[tid + NTH * i];
        if (ct == 0) {
            const float* const nst = slot_phi(s0 + sg) + (size_t)K * K;
#pragma unroll
            for (int j = 0; j < RPT; ++j) npre[j] = nst[(size_t)(VR * vt + rg + RG * j) * K + k];
        }
    };
    fetch(0, 0);
    for (int sg = 0; sg + 1 < nseg; ++sg) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) acc[j] = npre[j];
        for (int ct = 0; ct < NCT; ++ct) {
            __syncthreads();  // the previous tile (and the rows of s) have been read
#pragma unroll
            for (int i = 0; i < NLD; ++i) reinterpret_cast<f32x4*>(phs)[tid + NTH * i] = pre[i];
            __syncthreads();
            if (ct + 1 < NCT) fetch(sg, ct + 1);
            else if (sg + 2 < nseg) fetch(sg + 1, 0);
#pragma unroll 4
            for (int c = 0; c < CT; c += 4) {
                float pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[e] = phs[(c + e) * K + k];
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    const f32x4 sv = *reinterpret_cast<const f32x4*>(&s[rg + RG * j][ct * CT + c]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[j] = fmaf(sv[e], pk[e], acc[j]);
                }
            }
        }
        __syncthreads();  // every thread is done with s
        float* const nst = slot_phi(s0 + sg) + (size_t)K * K;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            s[rg + RG * j][k] = acc[j];
            nst[(size_t)(VR * vt + rg + RG * j) * K + k] = acc[j];
        }
    }
}

// K: compiled key width; V: value part width
template <typename T, int K, int V>
hipError_t launch_kv(ChunkArgs p, hipStream_t stream) {
    const int sl = p.L.seglen;
    const long long nch = chunk_bound(p.B, p.N);
    long long main_units = (long long)p.B * p.H * p.VS, sum_units = 0;
    if (sl != INT_MAX) {  // (one value part)
        main_units = (nch / sl + p.B) * p.H;
        sum_units = (nch / sl) * p.H;
    }
    // token rows are addressed through 32-bit buffer offsets within a chunk
    if ((p.x.sq > (1 << 23)) || (p.x.sk > (1 << 23)) || (p.x.sv > (1 << 23)) || (long long)CH * p.H * p.V > (1 << 29))
        return hipErrorInvalidConfiguration;
    const long long tm_blocks = nch * p.H;
    const long long comb_blocks = (long long)p.B * p.H * (V / 8);
    if (main_units > kMaxBlocks || comb_blocks > kMaxBlocks || tm_blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(1024), 0, stream, p);
    if (p.N > 0) {
        p.n_blocks = (int)tm_blocks;
        hipLaunchKernelGGL((chunk_tmat_kernel<T, K>), dim3((unsigned)tm_blocks), dim3(256), 0, stream, p);
    }
    constexpr int VTW = kValueTilesPerWave;
    constexpr int NT = 64 * (V / (16 * VTW));
    if constexpr (chunk_segments_ok(K, V, 1)) {
        if (sum_units > 0) {
            p.n_blocks = (int)sum_units;
            hipLaunchKernelGGL((chunk_fused_kernel<T, K, V, kSummary, VTW>), dim3((unsigned)sum_units), dim3(NT), 0, stream, p);
            hipLaunchKernelGGL((chunk_combine_kernel<K, V>), dim3((unsigned)comb_blocks), dim3(combine_threads<K>()), 0, stream, p);
        }
    } else if (sum_units > 0) {
        return hipErrorInvalidConfiguration;  // (segments are never planned for these widths)
    }
    p.n_blocks = (int)main_units;
    if (p.cap > 0)
        hipLaunchKernelGGL((chunk_fused_kernel<T, K, V, kMainCapture, VTW>), dim3((unsigned)main_units), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((chunk_fused_kernel<T, K, V, kMain, VTW>), dim3((unsigned)main_units), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// The main, summary and combine kernels for one compiled key width K (both I/O types), dispatched
// on the value part width.  Each width is instantiated in a translation unit of its own.
template <typename T, int K>
hipError_t launch_chunk_kw(const ChunkArgs& p, hipStream_t stream) {
    switch (chunk_value_tile(p.V)) {
        case 32: return launch_kv<T, K, 32>(p, stream);
        case 64: return launch_kv<T, K, 64>(p, stream);
        default: return launch_kv<T, K, 128>(p, stream);
    }
}
#define GDN_CHUNK_INSTANTIATE(K)                                                    \
    template hipError_t launch_chunk_kw<BF16, K>(const ChunkArgs&, hipStream_t); \
    template hipError_t launch_chunk_kw<F16, K>(const ChunkArgs&, hipStream_t);
#define GDN_CHUNK_EXTERN(K)                                                                \
    extern template hipError_t launch_chunk_kw<BF16, K>(const ChunkArgs&, hipStream_t); \
    extern template hipError_t launch_chunk_kw<F16, K>(const ChunkArgs&, hipStream_t);

}  // namespace gdn
