// gdn_conv.hip -- varlen depthwise causal conv1d with a carried window (gfx950).
//
// Operation: paged_ssm.rs page, kernel string CONV (see gdn.h for the definition).  The page's
// kernel runs one thread per (sequence, channel), serial over the sequence.  Here the work is
// token-parallel instead, which is what fills 256 CUs for a single long sequence:
//
//   * a thread owns VEC adjacent channels (16 bytes of a token row: 8 half or 4 fp32 channels), so
//     every row access of a wave is one contiguous, fully coalesced segment;
//   * "body" blocks own a tile of TT consecutive packed tokens and compute every token whose local
//     index is >= L (all taps then fall inside the sequence); for dilation 1 the W taps slide
//     through registers, so each token row is loaded once;
//   * "head" blocks own one sequence: they compute its first min(L + kHeadExtra, len) tokens -- the
//     first L are the only ones whose taps reach into the carried window; the few after them make a
//     short sequence (a decode or verification step) a head block's work alone -- and then write
//     the new window.  The window is
//     read and written by the same thread in that order, so state_out may alias state_in;
//   * with capture (speculative decoding: paged_ssm.rs page, CONV_CAPTURE_INIT / _STEP) the head
//     blocks also copy the sequence's first captured token rows into its update slots and zero the
//     slots after them.
//
// Every block checks the whole offsets array first and writes nothing when it is malformed; the
// offsets are staged in LDS on the way (up to kStagedOffsets entries), so that body blocks map their
// tokens to sequences without chains of dependent global loads.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int kConvTile = 16;        // tokens per body block
constexpr int kHeadExtra = 8;        // tokens a head block computes beyond the first L
constexpr int kStagedOffsets = 2048;  // offsets kept in LDS when B + 1 fits

struct ConvArgs {
    const void* x;
    const void* w;
    const void* bias;
    const void* state_in;  // not restrict: may alias state_out
    void* y;
    void* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    int B, N, C, D, L;
    int silu;
    int n_cvec;  // C / VEC
    int n_cblk;  // channel blocks per item
    int tile;    // tokens per body block
    int cap;                // capture slots per sequence (0 = no capture)
    const int32_t* counts;  // [B] tokens to capture
    void* updates;          // [B, cap, C] x dtype
};

template <typename T, int VEC>
__device__ __forceinline__ void load_row(const typename T::storage* p, float (&v)[VEC]) {
    if constexpr (VEC == 1) {
        v[0] = to_f32<T>(p[0]);
    } else {
        static_assert(VEC * sizeof(typename T::storage) == 16, "one 16-byte vector per thread");
        const u32x4 raw = *reinterpret_cast<const u32x4*>(p);
        if constexpr (std::is_same<T, F32>::value) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(raw[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = to_f32<T>((uint16_t)(raw[i] & 0xffffu));
                v[2 * i + 1] = to_f32<T>((uint16_t)(raw[i] >> 16));
            }
        }
    }
}

template <typename T, int VEC>
__device__ __forceinline__ void store_row(typename T::storage* p, const float (&v)[VEC]) {
    if constexpr (VEC == 1) {
        p[0] = from_f32<T>(v[0]);
    } else {
        u32x4 raw;
        if constexpr (std::is_same<T, F32>::value) {
#pragma unroll
            for (int i = 0; i < 4; ++i) raw[i] = __float_as_uint(v[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                raw[i] = (uint32_t)from_f32<T>(v[2 * i]) | ((uint32_t)from_f32<T>(v[2 * i + 1]) << 16);
        }
        *reinterpret_cast<u32x4*>(p) = raw;
    }
}

// Element i of a 16-byte row vector, as raw storage.
template <typename T>
__device__ __forceinline__ typename T::storage raw_elem(const u32x4& raw, int i) {
    if constexpr (std::is_same<T, F32>::value) return __uint_as_float(raw[i]);
    else return (uint16_t)((raw[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}

// Capture of sequence b by the thread owning channels c0 .. c0+VEC-1: slot i < captured holds the
// raw row x[start + i] (bit copy), the remaining slots zeros.
template <typename T, int VEC>
__device__ __forceinline__ void capture_rows(const ConvArgs& p, int b, int start, int len, int c0) {
    using TS = typename T::storage;
    const int n = captured_tokens(p.counts, nullptr, p.cap, b, len);
    const TS* x = static_cast<const TS*>(p.x);
    TS* u = static_cast<TS*>(p.updates) + (size_t)b * p.cap * p.C + c0;
    for (int i = 0; i < p.cap; ++i) {
        if constexpr (VEC > 1) {
            const u32x4 v = i < n ? *reinterpret_cast<const u32x4*>(x + (size_t)(start + i) * p.C + c0)
                                  : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(u + (size_t)i * p.C) = v;
        } else {
            u[(size_t)i * p.C] = i < n ? x[(size_t)(start + i) * p.C + c0] : (TS)0;
        }
    }
}

// The whole-call offsets check of offsets_malformed, storing each entry into s_off on the way when
// s_off is given.  Ends with a block barrier, after which s_off is complete.
__device__ __forceinline__ bool check_stage_offsets(const int32_t* __restrict__ offsets, int B, int N, int* s_off) {
    int bad = 0;
    for (int i = threadIdx.x; i <= B; i += blockDim.x) {
        const int o = offsets[i];
        if (s_off != nullptr) s_off[i] = o;
        if (i == 0) bad |= (o != 0);
        else bad |= (offsets[i - 1] > o);
        if (i == B) bad |= (o != N);
    }
    return __syncthreads_or(bad) != 0;
}

// SiLU z / (1 + e^-z) with the hardware exp2 and reciprocal (each within a couple of ulp of fp32):
// the IEEE-exact expf and division cost ~35 VALU instructions per element and made the conv
// arithmetic-bound.  z -> -inf gives e^-z = inf, rcp(inf) = 0 and an output of -0 (the limit).
template <int VEC>
__device__ __forceinline__ void activate(float (&acc)[VEC], int silu) {
    if (silu) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = acc[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-acc[i]));
    }
}

// T: element type of x, w, bias, y.  S: element type of the window (T or F32).
template <typename T, typename S, int VEC, int W>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs p) {
    using TS = typename T::storage;
    using SS = typename S::storage;
    __shared__ int s_off[kStagedOffsets];
    const bool staged = p.B < kStagedOffsets;
    const bool malformed = check_stage_offsets(p.offsets, p.B, p.N, staged ? s_off : nullptr);
    report_status(p.dev_status, malformed);
    if (malformed) return;
    auto off = [&](int i) { return staged ? s_off[i] : p.offsets[i]; };
    // sequence containing token t (t < N): the last b with off(b) <= t
    auto find_seq = [&](int t) {
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off(mid) <= t) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };

    const int item = (int)(blockIdx.x / (unsigned)p.n_cblk);
    const int cvec = (int)(blockIdx.x % (unsigned)p.n_cblk) * (int)blockDim.x + (int)threadIdx.x;
    if (cvec >= p.n_cvec) return;
    const int C = p.C, D = p.D, L = p.L;

    // Body blocks: which tokens of the tile have local index >= L + kHeadExtra (the rest belong to
    // head blocks).  A tile without any -- every tile of a batch of short sequences -- ends here,
    // before any load.
    unsigned body_mask = 0;
    if (item >= p.B) {
        const int t0 = (item - p.B) * p.tile;
        const int t1 = min(t0 + p.tile, p.N);
        int b = find_seq(t0);
        int next = off(b + 1);
        for (int t = t0; t < t1; ++t) {
            while (next <= t) {
                ++b;
                next = off(b + 1);
            }
            if (t - off(b) >= L + kHeadExtra) body_mask |= 1u << (t - t0);
        }
        if (body_mask == 0) return;
    }
    const int c0 = cvec * VEC;
    const TS* __restrict__ x = static_cast<const TS*>(p.x);
    TS* __restrict__ y = static_cast<TS*>(p.y);

    float wr[VEC][W];
    {
        const TS* wp = static_cast<const TS*>(p.w) + (size_t)c0 * W;
        if constexpr (VEC > 1) {
            // the thread's VEC*W weights are contiguous and 16-byte aligned: W vector loads
            union {
                u32x4 v[W];
                TS e[VEC * W];
            } u;
#pragma unroll
            for (int k = 0; k < W; ++k) u.v[k] = reinterpret_cast<const u32x4*>(wp)[k];
#pragma unroll
            for (int i = 0; i < VEC; ++i)
#pragma unroll
                for (int j = 0; j < W; ++j) wr[i][j] = to_f32<T>(u.e[i * W + j]);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
#pragma unroll
                for (int j = 0; j < W; ++j) wr[i][j] = to_f32<T>(wp[i * W + j]);
        }
    }
    float bias[VEC];
    if (p.bias != nullptr) {
        load_row<T, VEC>(static_cast<const TS*>(p.bias) + c0, bias);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) bias[i] = 0.0f;
    }

    if constexpr (VEC > 1 && W > 1) {
      if (item < p.B && D == 1) {
        // ---- head, dilation 1: the thread's window block (VEC channels x L entries, contiguous) is
        // held in registers; L = W-1 is a compile-time size.  In a block whose threads are all live,
        // the block's whole window range (contiguous in memory) moves between HBM and LDS with
        // consecutive 16-byte accesses per lane, and each thread takes its block from LDS: a thread's
        // own block is VEC*L entries wide, so direct per-thread vector accesses would stride lanes
        // that far apart and cost several memory requests per lane.
        constexpr int L1 = W - 1;
        constexpr int NE = VEC * L1;                           // window elements of this thread
        constexpr int NCH = NE * (int)sizeof(SS) / 16;         // 16-byte chunks
        static_assert(NE * sizeof(SS) % 16 == 0, "window block is whole 16-byte chunks");
        __shared__ u32x4 s_win[256 * NCH];
        const int nthr = (int)blockDim.x, tid = (int)threadIdx.x;
        const bool full_block = ((int)(blockIdx.x % (unsigned)p.n_cblk) + 1) * nthr <= p.n_cvec;  // block-uniform
        const int b = item;
        const int start = off(b);
        const int len = off(b + 1) - start;
        const size_t wrow = ((size_t)b * C + c0) * (size_t)L1;  // window of channel c0 + i at wrow + i*L1
        // the block's window range, in 16-byte chunks, starts where thread 0's block does
        const size_t wblk = (((size_t)b * C + (size_t)(cvec - tid) * VEC) * (size_t)L1 * sizeof(SS)) / 16;
        union {
            u32x4 v[NCH];
            SS e[NE];
        } win;
        if (p.state_in != nullptr && full_block) {
            const u32x4* src = reinterpret_cast<const u32x4*>(p.state_in) + wblk;
#pragma unroll
            for (int k = 0; k < NCH; ++k) s_win[k * nthr + tid] = src[k * nthr + tid];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NCH; ++k) win.v[k] = s_win[tid * NCH + k];
        } else if (p.state_in != nullptr) {
            const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const SS*>(p.state_in) + wrow);
#pragma unroll
            for (int k = 0; k < NCH; ++k) win.v[k] = src[k];
        } else {
#pragma unroll
            for (int k = 0; k < NCH; ++k) win.v[k] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int l = 0; l < L1 + kHeadExtra; ++l) {
            if (l >= len) break;
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = bias[i];
#pragma unroll
            for (int j = 0; j < W; ++j) {
                const int m = l + j - L1;  // tap j of local token l (dilation 1)
                float xv[VEC];
                if (m >= 0) {
                    load_row<T, VEC>(x + (size_t)(start + m) * C + c0, xv);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) xv[i] = to_f32<S>(win.e[i * L1 + L1 + m]);
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] = fmaf(wr[i][j], xv[i], acc[i]);
            }
            activate<VEC>(acc, p.silu);
            store_row<T, VEC>(y + (size_t)(start + l) * C + c0, acc);
        }
        if (p.state_out != nullptr) {
            // new window entry j = old entry len + j while that exists, else token len - L1 + j
            union {
                u32x4 v[NCH];
                SS e[NE];
            } nw;
#pragma unroll
            for (int j = 0; j < L1; ++j) {
                const int src = len + j;
                u32x4 xr = u32x4{0u, 0u, 0u, 0u};
                if (src >= L1) xr = *reinterpret_cast<const u32x4*>(x + (size_t)(start + src - L1) * C + c0);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    SS v;
                    if constexpr (std::is_same<S, T>::value) v = raw_elem<T>(xr, i);
                    else v = to_f32<T>(raw_elem<T>(xr, i));  // exact widening into an fp32 window
#pragma unroll
                    for (int k = 0; k < L1; ++k)
                        if (src == k) v = win.e[i * L1 + k];
                    nw.e[i * L1 + j] = v;
                }
            }
            if (full_block) {
                // a thread reads and writes only its own block of s_win after the load barrier; the
                // barrier below hands the blocks to the threads that store them
#pragma unroll
                for (int k = 0; k < NCH; ++k) s_win[tid * NCH + k] = nw.v[k];
                __syncthreads();
                u32x4* dst = reinterpret_cast<u32x4*>(p.state_out) + wblk;
#pragma unroll
                for (int k = 0; k < NCH; ++k) dst[k * nthr + tid] = s_win[k * nthr + tid];
            } else {
                u32x4* dst = reinterpret_cast<u32x4*>(static_cast<SS*>(p.state_out) + wrow);
#pragma unroll
                for (int k = 0; k < NCH; ++k) dst[k] = nw.v[k];
            }
        }
        if (p.cap > 0) capture_rows<T, VEC>(p, b, start, len, c0);
        return;
      }
    }

    if (item < p.B) {
        // ---- head: the first min(L + kHeadExtra, len) tokens of sequence b, then the new window -----
        const int b = item;
        const int start = off(b);
        const int len = off(b + 1) - start;
        const SS* st_in = static_cast<const SS*>(p.state_in);
        SS* st_out = static_cast<SS*>(p.state_out);
        const size_t wrow = ((size_t)b * C + c0) * (size_t)L;  // window of channel c0 + i at wrow + i*L
        const int nh = len < L + kHeadExtra ? len : L + kHeadExtra;
        for (int l = 0; l < nh; ++l) {
            float acc[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = bias[i];
#pragma unroll
            for (int j = 0; j < W; ++j) {
                const int m = l - (W - 1 - j) * D;
                float xv[VEC];
                if (m >= 0) {
                    load_row<T, VEC>(x + (size_t)(start + m) * C + c0, xv);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        xv[i] = st_in ? to_f32<S>(st_in[wrow + (size_t)i * L + (L + m)]) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] = fmaf(wr[i][j], xv[i], acc[i]);
            }
            activate<VEC>(acc, p.silu);
            store_row<T, VEC>(y + (size_t)(start + l) * C + c0, acc);
        }
        if (st_out != nullptr) {
            // new window: entry j is xv(len - L + j); reading index len + j >= j of the old window
            // before writing index j keeps an aliased (in-place) update correct.
            for (int j = 0; j < L; ++j) {
                const int m = len - L + j;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    SS v;
                    if (m >= 0) {
                        const TS xs = x[(size_t)(start + m) * C + c0 + i];
                        if constexpr (std::is_same<S, T>::value) v = xs;
                        else v = to_f32<T>(xs);  // exact widening into an fp32 window
                    } else {
                        v = st_in ? st_in[wrow + (size_t)i * L + (L + m)] : (SS)0;
                    }
                    st_out[wrow + (size_t)i * L + j] = v;
                }
            }
        }
        if (p.cap > 0) capture_rows<T, VEC>(p, b, start, len, c0);
        return;
    }

    // ---- body: tokens [t0, t1) with local index >= L + kHeadExtra ---------------------------------
    if constexpr (VEC > 1 && W > 1) {
        if (D == 1) {
            // dilation 1: all TILE + L rows of the tile are loaded up front (independent 16-byte loads
            // in flight together), then every token reads its W taps from registers
            constexpr int L1 = W - 1;
            const int t0 = (item - p.B) * kConvTile;
            const int t1 = min(t0 + kConvTile, p.N);
            u32x4 rows[kConvTile + L1];
#pragma unroll
            for (int r = 0; r < kConvTile + L1; ++r) {
                const int t = t0 - L1 + r;
                rows[r] = (t >= 0 && t < t1) ? *reinterpret_cast<const u32x4*>(x + (size_t)t * C + c0) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < kConvTile; ++i) {
                const int t = t0 + i;
                if (!(body_mask & (1u << i))) continue;
                float acc[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = bias[e];
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    const u32x4 raw = rows[i + j];  // token t - (W-1-j)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = fmaf(wr[e][j], to_f32<T>(raw_elem<T>(raw, e)), acc[e]);
                }
                activate<VEC>(acc, p.silu);
                store_row<T, VEC>(y + (size_t)t * C + c0, acc);
            }
            return;
        }
    }
    const int t0 = (item - p.B) * p.tile;
    const int t1 = min(t0 + p.tile, p.N);
    float ring[W][VEC];  // ring[j] = x[t - (W-1-j)*D]
    int ring_t = -2;
    for (int t = t0; t < t1; ++t) {
        if (!(body_mask & (1u << (t - t0)))) continue;  // a head block's token
        if (D == 1 && ring_t == t - 1) {
#pragma unroll
            for (int j = 0; j + 1 < W; ++j)
#pragma unroll
                for (int i = 0; i < VEC; ++i) ring[j][i] = ring[j + 1][i];
            load_row<T, VEC>(x + (size_t)t * C + c0, ring[W - 1]);
        } else {
#pragma unroll
            for (int j = 0; j < W; ++j) load_row<T, VEC>(x + (size_t)(t - (W - 1 - j) * D) * C + c0, ring[j]);
        }
        ring_t = t;
        float acc[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = bias[i];
#pragma unroll
        for (int j = 0; j < W; ++j)
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[i] = fmaf(wr[i][j], ring[j][i], acc[i]);
        activate<VEC>(acc, p.silu);
        store_row<T, VEC>(y + (size_t)t * C + c0, acc);
    }
}

// ---- any width: the compiled kernels above hold the W taps in registers (W <= 8); wider convs
// take two plain kernels with the same arithmetic in the same order (bias, then the taps, fp32 FMA,
// the same SiLU and rounding).  The outputs first, one thread per (token, channel), reading the old
// window; then, in stream order, one thread per (sequence, channel) writes the new window in
// increasing entry order (reading entry j + len >= j before writing j, so an aliased window is
// correct) and the capture slots.
template <typename T, typename S>
__global__ __launch_bounds__(256) void conv_wide_out_kernel(ConvArgs p, int W) {
    using TS = typename T::storage;
    using SS = typename S::storage;
    __shared__ int s_off[kStagedOffsets];
    const bool staged = p.B < kStagedOffsets;
    const bool malformed = check_stage_offsets(p.offsets, p.B, p.N, staged ? s_off : nullptr);
    report_status(p.dev_status, malformed);
    if (malformed) return;
    auto off = [&](int i) { return staged ? s_off[i] : p.offsets[i]; };
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)p.N * p.C) return;
    const int C = p.C, D = p.D, L = p.L;
    const int t = (int)(idx / C), c = (int)(idx % C);
    int lo = 0, hi = p.B - 1;  // the sequence of token t: the last b with off(b) <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off(mid) <= t) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo, start = off(b), l = t - start;
    const TS* x = static_cast<const TS*>(p.x);
    const TS* w = static_cast<const TS*>(p.w) + (size_t)c * W;
    const SS* st_in = static_cast<const SS*>(p.state_in);
    const size_t wrow = ((size_t)b * C + c) * (size_t)L;
    float acc[1] = {p.bias != nullptr ? to_f32<T>(static_cast<const TS*>(p.bias)[c]) : 0.0f};
    for (int j = 0; j < W; ++j) {
        const int m = l - (W - 1 - j) * D;
        const float xv = m >= 0 ? to_f32<T>(x[(size_t)(start + m) * C + c])
                                : (st_in ? to_f32<S>(st_in[wrow + (size_t)(L + m)]) : 0.0f);
        acc[0] = fmaf(to_f32<T>(w[j]), xv, acc[0]);
    }
    activate<1>(acc, p.silu);
    static_cast<TS*>(p.y)[(size_t)t * C + c] = from_f32<T>(acc[0]);
}

template <typename T, typename S>
__global__ __launch_bounds__(256) void conv_wide_window_kernel(ConvArgs p) {
    using TS = typename T::storage;
    using SS = typename S::storage;
    const bool malformed = check_stage_offsets(p.offsets, p.B, p.N, nullptr);
    report_status(p.dev_status, malformed);  // (also when there are no tokens and no output launch)
    if (malformed) return;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)p.B * p.C) return;
    const int C = p.C, L = p.L;
    const int b = (int)(idx / C), c = (int)(idx % C);
    const int start = p.offsets[b], len = p.offsets[b + 1] - start;
    const TS* x = static_cast<const TS*>(p.x);
    const SS* st_in = static_cast<const SS*>(p.state_in);
    SS* st_out = static_cast<SS*>(p.state_out);
    const size_t wrow = ((size_t)b * C + c) * (size_t)L;
    if (st_out != nullptr) {
        for (int j = 0; j < L; ++j) {
            const int m = len - L + j;
            SS v;
            if (m >= 0) {
                const TS xs = x[(size_t)(start + m) * C + c];
                if constexpr (std::is_same<S, T>::value) v = xs;
                else v = to_f32<T>(xs);  // exact widening into an fp32 window
            } else {
                v = st_in ? st_in[wrow + (size_t)(L + m)] : (SS)0;
            }
            st_out[wrow + j] = v;
        }
    }
    if (p.cap > 0) {
        const int n = captured_tokens(p.counts, nullptr, p.cap, b, len);
        TS* u = static_cast<TS*>(p.updates) + (size_t)b * p.cap * C + c;
        for (int i = 0; i < p.cap; ++i) u[(size_t)i * C] = i < n ? x[(size_t)(start + i) * C + c] : (TS)0;
    }
}

template <typename T, typename S>
hipError_t launch_wide(const ConvArgs& p, int W, hipStream_t stream) {
    const long long out_blocks = ((long long)p.N * p.C + 255) / 256;
    const long long win_blocks = ((long long)p.B * p.C + 255) / 256;
    if (out_blocks > kMaxBlocks || win_blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    if (out_blocks > 0)
        hipLaunchKernelGGL((conv_wide_out_kernel<T, S>), dim3((unsigned)out_blocks), dim3(256), 0, stream, p, W);
    hipLaunchKernelGGL((conv_wide_window_kernel<T, S>), dim3((unsigned)win_blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T, typename S, int VEC>
hipError_t launch_vec(const ConvLaunch& a, hipStream_t stream) {
    ConvArgs p;
    p.x = a.x;
    p.w = a.w;
    p.bias = a.bias;
    p.state_in = a.state_in;
    p.y = a.y;
    p.state_out = a.state_out;
    p.offsets = a.offsets;
    p.dev_status = a.dev_status;
    p.B = a.B;
    p.N = a.N;
    p.C = a.C;
    p.D = a.D;
    p.L = (a.W - 1) * a.D;
    p.silu = a.silu ? 1 : 0;
    p.cap = a.cap;
    p.counts = a.counts;
    p.updates = a.updates;
    p.n_cvec = a.C / VEC;
    const int threads = p.n_cvec >= 256 ? 256 : ((p.n_cvec + 63) / 64) * 64;
    p.n_cblk = (p.n_cvec + threads - 1) / threads;
    p.tile = kConvTile;
    if (a.W > 8) return launch_wide<T, S>(p, a.W, stream);
    const long long n_tiles = ((long long)a.N + p.tile - 1) / p.tile;
    const long long blocks = ((long long)a.B + n_tiles) * p.n_cblk;
    if (blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    switch (a.W) {
#define GDN_CONV_CASE(WW)                                                                                    \
    case WW:                                                                                                 \
        hipLaunchKernelGGL((conv_kernel<T, S, VEC, WW>), dim3((unsigned)blocks), dim3(threads), 0, stream, p); \
        break;
        GDN_CONV_CASE(1)
        GDN_CONV_CASE(2)
        GDN_CONV_CASE(3)
        GDN_CONV_CASE(4)
        GDN_CONV_CASE(5)
        GDN_CONV_CASE(6)
        GDN_CONV_CASE(7)
        GDN_CONV_CASE(8)
#undef GDN_CONV_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_typed(const ConvLaunch& a, hipStream_t stream) {
    constexpr int VEC = 16 / (int)sizeof(typename T::storage);
    if (a.C % VEC == 0) return launch_vec<T, S, VEC>(a, stream);
    return launch_vec<T, S, 1>(a, stream);
}

}  // namespace

hipError_t launch_conv(const ConvLaunch& a, hipStream_t stream) {
    const int xs = a.x_dtype, ss = a.state_dtype;
    if (xs == GDN_F32) return launch_typed<F32, F32>(a, stream);
    if (xs == GDN_BF16) return ss == GDN_F32 ? launch_typed<BF16, F32>(a, stream) : launch_typed<BF16, BF16>(a, stream);
    if (xs == GDN_F16) return ss == GDN_F32 ? launch_typed<F16, F32>(a, stream) : launch_typed<F16, F16>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
