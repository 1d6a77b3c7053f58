// gdn_api.cpp -- the extern "C" entry points of libgdn: argument validation, path selection and
// dispatch to the kernel launchers.  Every check here runs on the host before anything is queued,
// so a rejected call launches nothing and writes nothing.  The checks mirror the claim predicates
// and handler checks of the paged_ssm.rs page (conv_claim, delta_claim, conv(), delta()):
// positive geometry, H divisible by HQ, key width at most 256, dtype agreement, int32-sized
// dispatches.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

bool dtype_ok(int d) { return d == GDN_F32 || d == GDN_BF16 || d == GDN_F16; }
long long dsize(int d) { return d == GDN_F32 ? 4 : 2; }
bool misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

gdn_status from_hip(hipError_t e) {
    if (e == hipSuccess) return GDN_OK;
    if (e == hipErrorInvalidConfiguration) return GDN_ERR_OVERFLOW;
    return GDN_ERR_HIP;
}

// Shape, dtype and flag checks shared by prepare, scan and the workspace query.
gdn_status check_scan_desc(const gdn_scan_desc* d) {
    if (d == nullptr) return GDN_ERR_NULL;
    if (d->B < 1 || d->N < 0 || d->HQ < 1 || d->H < 1 || d->K < 1 || d->V < 1) return GDN_ERR_SHAPE;
    if (d->H % d->HQ != 0 || d->K > 256) return GDN_ERR_SHAPE;
    if (!dtype_ok(d->qkv_dtype)) return GDN_ERR_DTYPE;
    if (d->gate_dtype != GDN_F32 && d->gate_dtype != d->qkv_dtype) return GDN_ERR_DTYPE;
    if (d->flags & ~(uint32_t)(GDN_L2NORM | GDN_SOFTPLUS | GDN_SIGMOID | GDN_NO_RETRIEVE | GDN_GATE_PER_KEY))
        return GDN_ERR_UNSUPPORTED;
    const long long C = 2ll * d->HQ * d->K + (long long)d->H * d->V;
    if (C > INT_MAX) return GDN_ERR_OVERFLOW;
    if ((long long)d->B * d->H > INT_MAX) return GDN_ERR_OVERFLOW;
    if (d->path < GDN_PATH_AUTO || d->path > GDN_PATH_CHUNK) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

// The packed [q | k | v] row as three token streams; its rows must start 16-byte aligned.
gdn_status packed_streams(const gdn_scan_desc* d, const void* qkv, gdn::TokenStreams* x) {
    const long long C = 2ll * d->HQ * d->K + (long long)d->H * d->V;
    if ((C * dsize(d->qkv_dtype)) % 16 != 0) return GDN_ERR_ALIGN;
    if (misaligned(qkv)) return GDN_ERR_ALIGN;
    const char* base = static_cast<const char*>(qkv);
    const long long es = dsize(d->qkv_dtype);
    x->q = qkv;
    x->k = base ? base + (long long)d->HQ * d->K * es : nullptr;
    x->v = base ? base + 2ll * d->HQ * d->K * es : nullptr;
    x->sq = x->sk = x->sv = C;
    return GDN_OK;
}

// Separate token streams: each used stream present (when there are tokens), 16-byte aligned, with
// a row stride of at least its row width whose rows all start 16-byte aligned.
gdn_status strided_streams(const gdn_scan_desc* d, const gdn_qkv_streams* s, bool need_qk, bool need_v,
                           gdn::TokenStreams* x) {
    if (s == nullptr) return GDN_ERR_NULL;
    const long long es = dsize(d->qkv_dtype);
    const long long wqk = (long long)d->HQ * d->K, wv = (long long)d->H * d->V;
    struct {
        const void* p;
        long long stride, width;
        bool used;
    } st[3] = {{s->q, s->q_stride, wqk, need_qk}, {s->k, s->k_stride, wqk, need_qk}, {s->v, s->v_stride, wv, need_v}};
    for (const auto& e : st) {
        if (!e.used) continue;
        if (d->N > 0 && e.p == nullptr) return GDN_ERR_NULL;
        if (e.stride < e.width) return GDN_ERR_SHAPE;
        if (d->N > 0 && e.stride > (LLONG_MAX / 4) / d->N) return GDN_ERR_OVERFLOW;
        if (misaligned(e.p) || (e.stride * es) % 16 != 0) return GDN_ERR_ALIGN;
    }
    x->q = need_qk ? s->q : nullptr;
    x->k = need_qk ? s->k : nullptr;
    x->v = need_v ? s->v : nullptr;
    x->sq = s->q_stride;
    x->sk = s->k_stride;
    x->sv = s->v_stride;
    return GDN_OK;
}

// The chunked path sums log-decays, so it needs every decay finite and positive (a decay input with
// the softplus gate), and it relies on normalised keys for a well-conditioned (I + A); it computes
// the gates and norms itself, so it runs on fused inputs only; its algebra is that of the rules
// with the retrieval term and one decay per head.  Built for bf16/fp16 I/O with K and V multiples
// of 8 (K at most 256).
// It records a capture from its first chunk, so at most 64 slots.  A call without tokens reads no
// decays (its chunked form only copies the initial states), so there the decay input may be absent.
bool chunk_eligible(const gdn_scan_desc* d, bool prepared, bool has_decay, int cap) {
    return !prepared && (has_decay || d->N == 0) && cap <= gdn::kChunkTokens && (d->flags & GDN_SOFTPLUS) &&
           (d->flags & GDN_L2NORM) &&
           !(d->flags & (GDN_NO_RETRIEVE | GDN_GATE_PER_KEY)) &&
           gdn::chunked_shape_supported(d->K, d->V, d->qkv_dtype);
}

// AUTO: DECODE for at most kDecodeShortTokens tokens per sequence on average (single tokens and
// short blocks stream the state once); past that CHUNK when eligible and the workspace suffices,
// SEQ otherwise.  The lengths themselves stay on the device, so the choice sees only N and B: at
// B = 256 (H = 32, K = V = 128) the chunked form ties SEQ at 12 tokens per sequence, is ahead from
// 16 on, and keeps a batch that mixes single tokens with one long prefill off the token-sequential
// chain of the long sequence (about 4.5x faster than SEQ with one 4096-token sequence).
int resolve_path(const gdn_scan_desc* d, bool prepared, bool has_decay, int cap, size_t ws_bytes) {
    if (d->path != GDN_PATH_AUTO) return d->path;
    if ((long long)d->N <= (long long)gdn::kDecodeShortTokens * d->B) return GDN_PATH_DECODE;
    if (chunk_eligible(d, prepared, has_decay, cap) &&
        ws_bytes >= gdn::chunked_workspace_bytes(d->B, d->N, d->HQ, d->H, d->K, d->V))
        return GDN_PATH_CHUNK;
    return GDN_PATH_SEQ;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "a dimension is out of range or inconsistent";
        case GDN_ERR_DTYPE: return "unknown or disallowed element type";
        case GDN_ERR_OVERFLOW: return "a size or launch grid exceeds the index range";
        case GDN_ERR_ALIGN: return "a tensor pointer or token row is not 16-byte aligned";
        case GDN_ERR_UNSUPPORTED: return "shape, flag or path not supported by this library";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "the HIP runtime rejected a launch";
        case GDN_ERR_OFFSETS: return "malformed offsets (device-detected; nothing written)";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// gdn_conv1d_varlen with an optional capture (cap == 0: none; the capture arguments were checked).
gdn_status conv_call(const gdn_conv_desc* d, const void* x, const void* w, const void* bias, const void* state_in,
                     void* y, void* state_out, const int32_t* offsets, int cap, const int32_t* counts,
                     void* updates, int32_t* dev_status, hipStream_t stream) {
    if (d == nullptr || w == nullptr || offsets == nullptr) return GDN_ERR_NULL;
    if (d->B < 1 || d->N < 0 || d->C < 1 || d->W < 1 || d->D < 1) return GDN_ERR_SHAPE;
    if (d->N > 0 && (x == nullptr || y == nullptr)) return GDN_ERR_NULL;
    if (!dtype_ok(d->x_dtype)) return GDN_ERR_DTYPE;
    if (d->state_dtype != d->x_dtype && d->state_dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (d->flags & ~(uint32_t)GDN_CONV_SILU) return GDN_ERR_UNSUPPORTED;
    const long long L = (long long)(d->W - 1) * d->D;
    if (L > INT_MAX || (long long)d->B * d->C > INT_MAX) return GDN_ERR_OVERFLOW;
    if (misaligned(x) || misaligned(w) || misaligned(bias) || misaligned(state_in) || misaligned(y) ||
        misaligned(state_out))
        return GDN_ERR_ALIGN;
    gdn::ConvLaunch a;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.state_in = L > 0 ? state_in : nullptr;
    a.y = y;
    a.state_out = L > 0 ? state_out : nullptr;
    a.offsets = offsets;
    a.dev_status = dev_status;
    a.B = d->B;
    a.N = d->N;
    a.C = d->C;
    a.W = d->W;
    a.D = d->D;
    a.x_dtype = d->x_dtype;
    a.state_dtype = d->state_dtype;
    a.silu = (d->flags & GDN_CONV_SILU) != 0;
    a.cap = cap;
    a.counts = counts;
    a.updates = updates;
    return from_hip(gdn::launch_conv(a, stream));
}

}  // namespace

extern "C" {

gdn_status gdn_conv1d_varlen(const gdn_conv_desc* d, const void* x, const void* w, const void* bias,
                             const void* state_in, void* y, void* state_out, const int32_t* offsets,
                             int32_t* dev_status, hipStream_t stream) {
    return conv_call(d, x, w, bias, state_in, y, state_out, offsets, 0, nullptr, nullptr, dev_status, stream);
}

gdn_status gdn_conv1d_varlen_capture(const gdn_conv_desc* d, const void* x, const void* w, const void* bias,
                                     const void* state_in, void* y, void* state_out, const int32_t* offsets,
                                     int32_t cap, const int32_t* counts, void* updates, int32_t* dev_status,
                                     hipStream_t stream) {
    if (d == nullptr || counts == nullptr || updates == nullptr) return GDN_ERR_NULL;
    if (cap < 1) return GDN_ERR_SHAPE;
    if ((long long)cap * d->C > INT_MAX) return GDN_ERR_OVERFLOW;
    if (misaligned(updates)) return GDN_ERR_ALIGN;
    return conv_call(d, x, w, bias, state_in, y, state_out, offsets, cap, counts, updates, dev_status, stream);
}

}  // extern "C"

namespace {

// gdn_prepare_qk_gates on token streams x (already checked; q/k unread when qk_out is NULL).
gdn_status prepare_call(const gdn_scan_desc* d, const gdn::TokenStreams& x, const void* a, const void* b,
                        const float* A_log, const float* dt_bias, float* qk_out, float* gb_out, hipStream_t stream) {
    if (d->N == 0) return GDN_OK;
    gdn::PrepareLaunch p;
    p.x = x;
    p.a = a;
    p.b = b;
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.qk_out = qk_out;
    p.gb_out = gb_out;
    p.N = d->N;
    p.HQ = d->HQ;
    p.H = d->H;
    p.K = d->K;
    p.V = d->V;
    p.qkv_dtype = d->qkv_dtype;
    p.gate_dtype = d->gate_dtype;
    p.flags = d->flags;
    return from_hip(gdn::launch_prepare(p, stream));
}

// Checks shared by the two prepare entry points (everything but the token streams).
gdn_status check_prepare(const gdn_scan_desc* d, const void* a, const float* A_log, const float* dt_bias,
                         const float* qk_out, const float* gb_out) {
    const gdn_status st = check_scan_desc(d);
    if (st != GDN_OK) return st;
    if (d->flags & GDN_GATE_PER_KEY) return GDN_ERR_UNSUPPORTED;  // its gate plane is one decay per head
    if (d->N > 0 && qk_out == nullptr && gb_out == nullptr) return GDN_ERR_NULL;  // N = 0 writes nothing
    if (a != nullptr && (d->flags & GDN_SOFTPLUS) && (A_log == nullptr || dt_bias == nullptr)) return GDN_ERR_NULL;
    if (misaligned(qk_out) || misaligned(gb_out)) return GDN_ERR_ALIGN;
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prepare_qk_gates(const gdn_scan_desc* d, const void* qkv, const void* a, const void* b,
                                const float* A_log, const float* dt_bias, float* qk_out, float* gb_out,
                                hipStream_t stream) {
    gdn_status st = check_prepare(d, a, A_log, dt_bias, qk_out, gb_out);
    if (st != GDN_OK) return st;
    if (d->N > 0 && qkv == nullptr && qk_out != nullptr) return GDN_ERR_NULL;
    gdn::TokenStreams x;
    if ((st = packed_streams(d, qkv, &x)) != GDN_OK) return st;
    return prepare_call(d, x, a, b, A_log, dt_bias, qk_out, gb_out, stream);
}

gdn_status gdn_prepare_qk_gates_strided(const gdn_scan_desc* d, const gdn_qkv_streams* streams, const void* a,
                                        const void* b, const float* A_log, const float* dt_bias, float* qk_out,
                                        float* gb_out, hipStream_t stream) {
    gdn_status st = check_prepare(d, a, A_log, dt_bias, qk_out, gb_out);
    if (st != GDN_OK) return st;
    gdn::TokenStreams x;
    if ((st = strided_streams(d, streams, qk_out != nullptr, false, &x)) != GDN_OK) return st;
    return prepare_call(d, x, a, b, A_log, dt_bias, qk_out, gb_out, stream);
}

gdn_status gdn_scan_workspace_bytes(const gdn_scan_desc* d, size_t* bytes) {
    if (bytes == nullptr) return GDN_ERR_NULL;
    const gdn_status st = check_scan_desc(d);
    if (st != GDN_OK) return st;
    // Resolved as AUTO would with an unlimited workspace, assuming fused inputs with a decay input
    // and no capture.
    const int path = resolve_path(d, false, true, false, SIZE_MAX);
    *bytes = path == GDN_PATH_CHUNK ? gdn::chunked_workspace_bytes(d->B, d->N, d->HQ, d->H, d->K, d->V) : 0;
    return GDN_OK;
}

}  // extern "C"

namespace {

// gdn_scan_varlen with an optional capture (cap == 0: none; the capture arguments were checked).
// The token streams x were checked by the caller (packed or strided); the rest is checked here.
// The workspace is the caller's buffer, or, when `scratch` is given, the library's own device
// scratch of ws_bytes bytes, which is looked up only after every host check has passed and only
// when the resolved path uses a workspace.
gdn_status scan_call(const gdn_scan_desc* d, const gdn::TokenStreams& x, const float* qk_prep, const float* gb_prep,
                     const void* a, const void* b, const float* A_log, const float* dt_bias, const float* state_in,
                     void* out, float* state_out, const int32_t* offsets, int cap, const int32_t* counts,
                     const int32_t* active, float* capsule, void* workspace, size_t ws_bytes, int32_t* dev_status,
                     int32_t* path_used, hipStream_t stream, gdn::ScratchFn scratch = nullptr) {
    if (offsets == nullptr) return GDN_ERR_NULL;
    if (d->N > 0 && out == nullptr) return GDN_ERR_NULL;
    if ((qk_prep == nullptr) != (gb_prep == nullptr)) return GDN_ERR_NULL;
    const bool prepared = qk_prep != nullptr;
    if (!prepared && a != nullptr && (d->flags & GDN_SOFTPLUS) && (A_log == nullptr || dt_bias == nullptr))
        return GDN_ERR_NULL;
    if (d->flags & GDN_GATE_PER_KEY) {
        // decays per key channel are evaluated in-kernel from raw inputs; nothing records them
        if (prepared || cap > 0) return GDN_ERR_UNSUPPORTED;
        if (misaligned(a)) return GDN_ERR_ALIGN;
    }
    if (misaligned(qk_prep) || misaligned(gb_prep) || misaligned(state_in) || misaligned(out) ||
        misaligned(state_out) || misaligned(workspace))
        return GDN_ERR_ALIGN;
    const bool has_ws = workspace != nullptr || scratch != nullptr;
    const int path = resolve_path(d, prepared, a != nullptr, cap, has_ws ? ws_bytes : 0);
    if (path == GDN_PATH_CHUNK) {
        if (!chunk_eligible(d, prepared, a != nullptr, cap)) return GDN_ERR_UNSUPPORTED;
        if (!has_ws || ws_bytes < gdn::chunked_workspace_bytes(d->B, d->N, d->HQ, d->H, d->K, d->V))
            return GDN_ERR_WORKSPACE;
        if (scratch != nullptr) {
            const gdn_status ss = scratch(&workspace);
            if (ss != GDN_OK) return ss;
        }
    }
    gdn::ScanLaunch s;
    s.x = x;
    s.qk_prep = qk_prep;
    s.gb_prep = gb_prep;
    s.a = prepared ? nullptr : a;
    s.b = prepared ? nullptr : b;
    s.A_log = A_log;
    s.dt_bias = dt_bias;
    s.state_in = state_in;
    s.out = out;
    s.state_out = state_out;
    s.offsets = offsets;
    s.dev_status = dev_status;
    s.workspace = workspace;
    s.ws_bytes = ws_bytes;
    s.B = d->B;
    s.N = d->N;
    s.HQ = d->HQ;
    s.H = d->H;
    s.K = d->K;
    s.V = d->V;
    s.qkv_dtype = d->qkv_dtype;
    s.gate_dtype = d->gate_dtype;
    s.flags = d->flags;
    s.scale = d->scale != 0.0f ? d->scale : 1.0f / std::sqrt((float)d->K);  // zero: the default
    s.path = path;
    s.cap = cap;
    s.counts = counts;
    s.active = active;
    s.capsule = capsule;
    const hipError_t e = path == GDN_PATH_CHUNK  ? gdn::launch_scan_chunked(s, stream)
                         : path == GDN_PATH_SEQ ? gdn::launch_scan_seq(s, stream)
                                                : gdn::launch_scan_decode(s, stream);
    const gdn_status rs = from_hip(e);
    if (rs == GDN_OK && path_used != nullptr) *path_used = path;
    return rs;
}

}  // namespace

extern "C" {

gdn_status gdn_scan_varlen(const gdn_scan_desc* d, const void* qkv, const float* qk_prep, const float* gb_prep,
                           const void* a, const void* b, const float* A_log, const float* dt_bias,
                           const float* state_in, void* out, float* state_out, const int32_t* offsets,
                           void* workspace, size_t ws_bytes, int32_t* dev_status, int32_t* path_used,
                           hipStream_t stream) {
    gdn_status st = check_scan_desc(d);
    if (st != GDN_OK) return st;
    if (d->N > 0 && qkv == nullptr) return GDN_ERR_NULL;
    gdn::TokenStreams x;
    if ((st = packed_streams(d, qkv, &x)) != GDN_OK) return st;
    return scan_call(d, x, qk_prep, gb_prep, a, b, A_log, dt_bias, state_in, out, state_out, offsets, 0, nullptr,
                     nullptr, nullptr, workspace, ws_bytes, dev_status, path_used, stream);
}

}  // extern "C"

namespace gdn {

gdn_status scan_varlen_scratch(const gdn_scan_desc* d, const void* qkv, const float* qk_prep, const float* gb_prep,
                               const void* a, const void* b, const float* A_log, const float* dt_bias,
                               const float* state_in, void* out, float* state_out, const int32_t* offsets,
                               ScratchFn scratch, size_t scratch_bytes, int32_t* dev_status, int32_t* path_used,
                               hipStream_t stream) {
    gdn_status st = check_scan_desc(d);
    if (st != GDN_OK) return st;
    if (d->N > 0 && qkv == nullptr) return GDN_ERR_NULL;
    gdn::TokenStreams x;
    if ((st = packed_streams(d, qkv, &x)) != GDN_OK) return st;
    return scan_call(d, x, qk_prep, gb_prep, a, b, A_log, dt_bias, state_in, out, state_out, offsets, 0, nullptr,
                     nullptr, nullptr, nullptr, scratch_bytes, dev_status, path_used, stream, scratch);
}

}  // namespace gdn

extern "C" {

gdn_status gdn_scan_varlen_strided(const gdn_scan_desc* d, const gdn_qkv_streams* streams, const float* qk_prep,
                                   const float* gb_prep, const void* a, const void* b, const float* A_log,
                                   const float* dt_bias, const float* state_in, void* out, float* state_out,
                                   const int32_t* offsets, void* workspace, size_t ws_bytes, int32_t* dev_status,
                                   int32_t* path_used, hipStream_t stream) {
    gdn_status st = check_scan_desc(d);
    if (st != GDN_OK) return st;
    gdn::TokenStreams x;  // prepared inputs replace q and k; v is always read
    if ((st = strided_streams(d, streams, qk_prep == nullptr, true, &x)) != GDN_OK) return st;
    return scan_call(d, x, qk_prep, gb_prep, a, b, A_log, dt_bias, state_in, out, state_out, offsets, 0, nullptr,
                     nullptr, nullptr, workspace, ws_bytes, dev_status, path_used, stream);
}

gdn_status gdn_scan_varlen_capture(const gdn_scan_desc* d, const void* qkv, const float* qk_prep,
                                   const float* gb_prep, const void* a, const void* b, const float* A_log,
                                   const float* dt_bias, const float* state_in, void* out, float* state_out,
                                   const int32_t* offsets, int32_t cap, const int32_t* counts, const int32_t* active,
                                   float* capsule, void* workspace, size_t ws_bytes, int32_t* dev_status,
                                   int32_t* path_used, hipStream_t stream) {
    const gdn_status st = check_scan_desc(d);
    if (st != GDN_OK) return st;
    if (counts == nullptr || capsule == nullptr) return GDN_ERR_NULL;
    if (cap < 1) return GDN_ERR_SHAPE;
    // the capsule row width must be an int32, as the pages' capsule geometry requires
    if ((long long)cap * ((long long)d->H + (long long)d->HQ * d->K + (long long)d->H * d->V) > INT_MAX)
        return GDN_ERR_OVERFLOW;
    if (misaligned(capsule)) return GDN_ERR_ALIGN;
    if (d->N > 0 && qkv == nullptr) return GDN_ERR_NULL;
    gdn::TokenStreams x;
    gdn_status ps = packed_streams(d, qkv, &x);
    if (ps != GDN_OK) return ps;
    return scan_call(d, x, qk_prep, gb_prep, a, b, A_log, dt_bias, state_in, out, state_out, offsets, cap, counts,
                     active, capsule, workspace, ws_bytes, dev_status, path_used, stream);
}

gdn_status gdn_decode_step(const gdn_conv_desc* cd, const gdn_scan_desc* sd, const void* x, const void* conv_w,
                           const void* conv_bias, const void* conv_state_in, void* conv_state_out, const void* a,
                           const void* b, const float* A_log, const float* dt_bias, const float* state_in, void* out,
                           float* state_out, const int32_t* offsets, int32_t* dev_status, hipStream_t stream) {
    if (cd == nullptr || conv_w == nullptr || offsets == nullptr) return GDN_ERR_NULL;
    const gdn_status st = check_scan_desc(sd);
    if (st != GDN_OK) return st;
    // token rows (packed [q | k | v], the conv output) must start 16-byte aligned
    if (((2ll * sd->HQ * sd->K + (long long)sd->H * sd->V) * dsize(sd->qkv_dtype)) % 16 != 0) return GDN_ERR_ALIGN;
    // the conv descriptor as gdn_conv1d_varlen checks it, and agreement with the scan descriptor
    if (cd->B < 1 || cd->N < 0 || cd->C < 1 || cd->W < 1 || cd->D < 1) return GDN_ERR_SHAPE;
    if (!dtype_ok(cd->x_dtype)) return GDN_ERR_DTYPE;
    if (cd->state_dtype != cd->x_dtype && cd->state_dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (cd->flags & ~(uint32_t)GDN_CONV_SILU) return GDN_ERR_UNSUPPORTED;
    if (cd->W > 8 || (long long)(cd->W - 1) * cd->D > INT_MAX) return GDN_ERR_UNSUPPORTED;
    if (cd->B != sd->B || cd->N != sd->N || (long long)cd->C != 2ll * sd->HQ * sd->K + (long long)sd->H * sd->V)
        return GDN_ERR_SHAPE;
    if (cd->x_dtype != sd->qkv_dtype) return GDN_ERR_DTYPE;
    // a decode step: at most one token per sequence (so N <= B; the device checks each length),
    // the recurrence on its DECODE path with fused inputs
    if (sd->N > sd->B) return GDN_ERR_UNSUPPORTED;
    if (sd->path != GDN_PATH_AUTO && sd->path != GDN_PATH_DECODE) return GDN_ERR_UNSUPPORTED;
    if (sd->flags & GDN_GATE_PER_KEY) return GDN_ERR_UNSUPPORTED;
    if (!gdn::decode_step_supported(sd->K, sd->V, sd->H / sd->HQ, cd->W, cd->D)) return GDN_ERR_UNSUPPORTED;
    if (sd->N > 0 && (x == nullptr || out == nullptr)) return GDN_ERR_NULL;
    if (a != nullptr && (sd->flags & GDN_SOFTPLUS) && (A_log == nullptr || dt_bias == nullptr)) return GDN_ERR_NULL;
    if (misaligned(x) || misaligned(conv_w) || misaligned(conv_bias) || misaligned(conv_state_in) ||
        misaligned(conv_state_out) || misaligned(state_in) || misaligned(out) || misaligned(state_out))
        return GDN_ERR_ALIGN;
    const bool has_window = cd->W > 1;
    gdn::DecodeStepLaunch l;
    l.x = x;
    l.conv_w = conv_w;
    l.conv_bias = conv_bias;
    l.conv_state_in = has_window ? conv_state_in : nullptr;
    l.conv_state_out = has_window ? conv_state_out : nullptr;
    l.a = a;
    l.b = b;
    l.A_log = A_log;
    l.dt_bias = dt_bias;
    l.state_in = state_in;
    l.out = out;
    l.state_out = state_out;
    l.offsets = offsets;
    l.dev_status = dev_status;
    l.B = sd->B;
    l.N = sd->N;
    l.HQ = sd->HQ;
    l.H = sd->H;
    l.K = sd->K;
    l.V = sd->V;
    l.W = cd->W;
    l.D = cd->D;
    l.qkv_dtype = sd->qkv_dtype;
    l.state_dtype = cd->state_dtype;
    l.gate_dtype = sd->gate_dtype;
    l.flags = sd->flags;
    l.silu = (cd->flags & GDN_CONV_SILU) != 0;
    l.scale = sd->scale != 0.0f ? sd->scale : 1.0f / std::sqrt((float)sd->K);  // zero: the default
    return from_hip(gdn::launch_decode_step(l, stream));
}

}  // extern "C"
