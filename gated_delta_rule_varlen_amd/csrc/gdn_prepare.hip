// gdn_prepare.hip -- q/k L2 normalisation plus decay and update-rate gates (gfx950).
//
// Operation: paged_ssm.rs page, kernel string DELTA_PREPARE; gate formulas also on the
// gated_delta_rate_activation.rs page (see gdn.h).  The page's kernel runs one 32-lane group per
// (token, value head) and normalises a key head's q/k inside it.  Here the [q | k] part of a token
// row is treated as 2*HQ rows of K contiguous elements: a row is owned by K/VEC lanes (VEC =
// elements per 16-byte load), so each wave reads and writes whole contiguous segments and the row's
// sum of squares is a DPP reduction inside the lane group.  The gates of all (token, value head)
// pairs are computed by extra blocks of the same launch (one launch, both outputs), with gate
// inputs widened to fp32 first.  HBM-bound: reads 2*HQ*K*s_x + 2*H*s_g bytes and writes
// (2*HQ*K + 2*H)*4 bytes per token.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

struct PrepArgs {
    TokenStreams x;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    float* qk_out;
    float* gb_out;
    int N, HQ, H, K;
    int gate_dtype;
    uint32_t flags;
    long long n_rows;   // N * 2 * HQ
    int n_row_blocks;   // blocks that normalise rows; the rest compute gates
};

// Gate and rate of token t, value head h (fused into the scan as well; see gdn_scan.hip).
__device__ __forceinline__ void gate_rate(const PrepArgs& p, long long i, int h, float& g, float& beta) {
    g = 1.0f;
    if (p.a != nullptr) {
        float x = load_any(p.a, p.gate_dtype, (size_t)i);
        if (p.flags & GDN_SOFTPLUS) x = -expf(p.A_log[h]) * softplus_f(x + p.dt_bias[h]);
        g = expf(x);
    }
    beta = 1.0f;
    if (p.b != nullptr) {
        beta = load_any(p.b, p.gate_dtype, (size_t)i);
        if (p.flags & GDN_SIGMOID) beta = 1.0f / (1.0f + expf(-beta));
    }
}

template <typename T, int K, bool KX>
__global__ __launch_bounds__(256) void prepare_kernel(PrepArgs p) {
    using TS = typename T::storage;
    // K is the compiled row width; rows are Kr wide (Kr < K: the lanes' elements past Kr read as
    // zero and are not written)
    const int Kr = KX ? K : p.K;
    constexpr int VEC = 16 / (int)sizeof(TS);  // elements per 16-byte load
    constexpr int RL = K / VEC;                // lanes per row
    static_assert(RL >= 1 && RL <= 64 && (RL & (RL - 1)) == 0, "row must map onto a power-of-two lane group");
    constexpr int ROWS = 256 / RL;             // rows per block

    if ((int)blockIdx.x < p.n_row_blocks) {
        if (p.qk_out == nullptr) return;
        const long long row = (long long)blockIdx.x * ROWS + threadIdx.x / RL;
        const int lane = threadIdx.x % RL;
        const bool live = row < p.n_rows;  // whole lane groups are live or dead together
        const long long rr = live ? row : 0;
        const long long t = rr / (2 * p.HQ);
        const int r = (int)(rr % (2 * p.HQ));  // 0..HQ-1: q rows, HQ..2HQ-1: k rows
        const TS* src = r < p.HQ ? static_cast<const TS*>(p.x.q) + (size_t)t * p.x.sq + (size_t)r * Kr
                                 : static_cast<const TS*>(p.x.k) + (size_t)t * p.x.sk + (size_t)(r - p.HQ) * Kr;
        float v[VEC];
        {
            const u32x4 raw = ld_raw16<TS, VEC, KX>(src, lane * VEC, Kr);
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
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) ss = fmaf(v[i], v[i], ss);
        ss = group_sum<RL>(ss);
        const float scale = (p.flags & GDN_L2NORM) ? rsqrtf(ss + 1e-12f) : 1.0f;
        if (!live) return;
        const int plane = r / p.HQ, hq = r % p.HQ;
        float* dst = p.qk_out + (((size_t)plane * p.N + (size_t)t) * p.HQ + hq) * Kr;
#pragma unroll
        for (int i = 0; i < VEC; i += 4)
            st_row4<KX, false>(dst, lane * VEC + i, Kr,
                               f32x4{v[i] * scale, v[i + 1] * scale, v[i + 2] * scale, v[i + 3] * scale});
        return;
    }
    if (p.gb_out == nullptr) return;
    const long long i = (long long)(blockIdx.x - p.n_row_blocks) * 256 + threadIdx.x;
    if (i >= (long long)p.N * p.H) return;
    const int h = (int)(i % p.H);
    float g, beta;
    gate_rate(p, i, h, g, beta);
    p.gb_out[i] = g;
    p.gb_out[(size_t)p.N * p.H + i] = beta;
}

template <typename T, int K, bool KX>
hipError_t launch_k(const PrepArgs& p0, hipStream_t stream) {
    PrepArgs p = p0;
    constexpr int VEC = 16 / (int)sizeof(typename T::storage);
    constexpr int ROWS = 256 / (K / VEC);
    p.n_row_blocks = p.qk_out ? (int)((p.n_rows + ROWS - 1) / ROWS) : 0;
    const long long gate_blocks = p.gb_out ? ((long long)p.N * p.H + 255) / 256 : 0;
    const long long blocks = p.n_row_blocks + gate_blocks;
    if (blocks == 0) return hipSuccess;
    if (blocks > kMaxBlocks) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prepare_kernel<T, K, KX>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const PrepArgs& p, hipStream_t stream) {
    switch (p.K) {
        case 32: return launch_k<T, 32, true>(p, stream);
        case 64: return launch_k<T, 64, true>(p, stream);
        case 128: return launch_k<T, 128, true>(p, stream);
        case 256: return launch_k<T, 256, true>(p, stream);
        default: break;
    }
    // any other width up to 256: the next of them, with the elements past K masked
    if (p.K < 1 || p.K > 256) return hipErrorInvalidValue;
    switch (padded_key_width(p.K)) {
        case 32: return launch_k<T, 32, false>(p, stream);
        case 64: return launch_k<T, 64, false>(p, stream);
        case 128: return launch_k<T, 128, false>(p, stream);
        default: return launch_k<T, 256, false>(p, stream);
    }
}

}  // namespace

hipError_t launch_prepare(const PrepareLaunch& a, hipStream_t stream) {
    PrepArgs p;
    p.x = a.x;
    p.a = a.a;
    p.b = a.b;
    p.A_log = a.A_log;
    p.dt_bias = a.dt_bias;
    p.qk_out = a.qk_out;
    p.gb_out = a.gb_out;
    p.N = a.N;
    p.HQ = a.HQ;
    p.H = a.H;
    p.K = a.K;
    p.gate_dtype = a.gate_dtype;
    p.flags = a.flags;
    p.n_rows = (long long)a.N * 2 * a.HQ;
    p.n_row_blocks = 0;
    switch (a.qkv_dtype) {
        case GDN_F32: return launch_t<F32>(p, stream);
        case GDN_BF16: return launch_t<BF16>(p, stream);
        case GDN_F16: return launch_t<F16>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
