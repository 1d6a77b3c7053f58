// gdn_chunk_k256.hip -- the chunked form's kernels at compiled key width 256 (keys 129 to 256).
#include "gdn_chunk.hpp"

namespace gdn {
GDN_CHUNK_INSTANTIATE(256)
}  // namespace gdn
