// gdn_chunk.hip -- host side of the chunked form: eligibility, workspace size and the launch,
// dispatched on the compiled key width (the kernels are in gdn_chunk.hpp and are instantiated in
// gdn_chunk_k64.hip, gdn_chunk_k128.hip and gdn_chunk_k256.hip).
// (only the shared definitions are used here; the kernels of the header are not emitted)
#pragma clang diagnostic ignored "-Wunneeded-internal-declaration"
#pragma clang diagnostic ignored "-Wunused-function"
#include "gdn_chunk.hpp"

namespace gdn {

GDN_CHUNK_EXTERN(64)
GDN_CHUNK_EXTERN(128)
GDN_CHUNK_EXTERN(256)

namespace {
template <typename T>
hipError_t launch_t(const ChunkArgs& p, hipStream_t stream) {
    switch (chunk_key_width(p.K)) {
        case 64: return launch_chunk_kw<T, 64>(p, stream);
        case 128: return launch_chunk_kw<T, 128>(p, stream);
        default: return launch_chunk_kw<T, 256>(p, stream);
    }
}
}  // namespace

// Half-precision I/O (the MFMA operands), key and value widths multiples of 8 (16-byte row pieces),
// keys at most 256.
bool chunked_shape_supported(int K, int V, int qkv_dtype) {
    return (qkv_dtype == GDN_BF16 || qkv_dtype == GDN_F16) && K >= 8 && K <= 256 && K % 8 == 0 && V >= 8 &&
           V % 8 == 0;
}

size_t chunked_workspace_bytes(int B, int N, int HQ, int H, int K, int V) {
    (void)HQ;
    return ws_layout(B, N, H, K, V).total;
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
    p.L = ws_layout(a.B, a.N, a.H, a.K, a.V);
    p.B = a.B;
    p.N = a.N;
    p.HQ = a.HQ;
    p.H = a.H;
    p.K = a.K;
    p.V = a.V;
    p.G = a.H / a.HQ;
    p.VS = chunk_value_parts(a.V);
    p.gate_dtype = a.gate_dtype;
    p.flags = a.flags;
    p.scale = a.scale;
    p.n_blocks = 0;
    p.cap = a.cap;
    p.counts = a.counts;
    p.active = a.active;
    p.capsule = a.capsule;
    if (a.qkv_dtype == GDN_BF16) return launch_t<BF16>(p, stream);
    if (a.qkv_dtype == GDN_F16) return launch_t<F16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
