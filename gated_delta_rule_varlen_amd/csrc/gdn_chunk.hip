// gdn_chunk.hip -- chunked (WY / UT-transform) form of the gated delta-rule recurrence (gfx950).
// Not built yet: the entry point rejects GDN_PATH_CHUNK before reaching this launcher.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

size_t chunked_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_scan_chunked(const ScanLaunch&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
