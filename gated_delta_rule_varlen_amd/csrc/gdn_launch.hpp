// gdn_launch.hpp -- host-side launchers of the libgdn kernels (internal; not part of the ABI).
// The entry points in gdn_api.cpp validate every argument and then call exactly one of these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

struct ConvLaunch {
    const void* x;
    const void* w;
    const void* bias;
    const void* state_in;
    void* y;
    void* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    int B, N, C, W, D;
    int x_dtype, state_dtype;
    bool silu;
    // capture (cap > 0): the first captured tokens' rows of x into updates [B, cap, C] x_dtype
    int cap;
    const int32_t* counts;
    void* updates;
};
hipError_t launch_conv(const ConvLaunch& a, hipStream_t stream);

// The token streams the recurrence reads: q and k rows (HQ*K elements per token) and v rows (H*V per
// token), each from its own base with its own row stride in elements.  A packed [q | k | v] row of
// width C = 2*HQ*K + H*V is the case q = qkv, k = qkv + HQ*K, v = qkv + 2*HQ*K, all strides C.
struct TokenStreams {
    const void* q;
    const void* k;
    const void* v;
    long long sq, sk, sv;
};

struct PrepareLaunch {
    TokenStreams x;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    float* qk_out;
    float* gb_out;
    int N, HQ, H, K, V;
    int qkv_dtype, gate_dtype;
    uint32_t flags;
};
hipError_t launch_prepare(const PrepareLaunch& a, hipStream_t stream);

struct ScanLaunch {
    TokenStreams x;
    const float* qk_prep;  // non-NULL selects the prepared variant
    const float* gb_prep;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    const float* state_in;
    void* out;
    float* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    void* workspace;
    size_t ws_bytes;
    int B, N, HQ, H, K, V;
    int qkv_dtype, gate_dtype;
    uint32_t flags;
    float scale;  // already resolved (> 0)
    int path;     // resolved: GDN_PATH_DECODE, GDN_PATH_SEQ or GDN_PATH_CHUNK
    // capture (cap > 0): g, k^ and delta of the first captured tokens into capsule
    // [B, cap*(H + HQ*K + H*V)] fp32; active (device, NULL = always) switches it off when 0
    int cap;
    const int32_t* counts;
    const int32_t* active;
    float* capsule;
};
hipError_t launch_scan_decode(const ScanLaunch& a, hipStream_t stream);  // DECODE
hipError_t launch_scan_seq(const ScanLaunch& a, hipStream_t stream);     // SEQ
hipError_t launch_scan_chunked(const ScanLaunch& a, hipStream_t stream);    // CHUNK
size_t chunked_workspace_bytes(int B, int N, int HQ, int H, int K, int V);

struct DecodeStepLaunch {
    const void* x;
    const void* conv_w;
    const void* conv_bias;
    const void* conv_state_in;
    void* conv_state_out;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    const float* state_in;
    void* out;
    float* state_out;
    const int32_t* offsets;
    int32_t* dev_status;
    int B, N, HQ, H, K, V, W, D;
    int qkv_dtype, state_dtype, gate_dtype;
    uint32_t flags;
    bool silu;
    float scale;  // already resolved (> 0)
};
hipError_t launch_decode_step(const DecodeStepLaunch& a, hipStream_t stream);
bool decode_step_supported(int K, int V, int G, int W, int D);
bool chunked_shape_supported(int K, int V, int qkv_dtype);

// Supplies the library's own device scratch for the current device (allocation-free entry points).
typedef gdn_status (*ScratchFn)(void** ptr);
// gdn_scan_varlen on a packed row with the workspace taken from `scratch` (scratch_bytes bytes).
gdn_status scan_varlen_scratch(const gdn_scan_desc* d, const void* qkv, const float* qk_prep, const float* gb_prep,
                               const void* a, const void* b, const float* A_log, const float* dt_bias,
                               const float* state_in, void* out, float* state_out, const int32_t* offsets,
                               ScratchFn scratch, size_t scratch_bytes, int32_t* dev_status, int32_t* path_used,
                               hipStream_t stream);

// Longest sequence the DECODE kernel carries column by column with staged token operands; AUTO
// takes DECODE while the average sequence is no longer than this.
constexpr int kDecodeShortTokens = 8;

// Tokens per chunk of the chunked form (it records a capture from a sequence's first chunk).
constexpr int kChunkTokens = 64;

// Limits of the launch grids (checked by the entry points before launching).
constexpr long long kMaxBlocks = (1ll << 31) - 1;

}  // namespace gdn
