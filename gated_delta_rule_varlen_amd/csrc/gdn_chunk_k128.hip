// gdn_chunk_k128.hip -- the chunked form's kernels at compiled key width 128 (keys 65 to 128).
#include "gdn_chunk.hpp"

namespace gdn {
GDN_CHUNK_INSTANTIATE(128)
}  // namespace gdn
