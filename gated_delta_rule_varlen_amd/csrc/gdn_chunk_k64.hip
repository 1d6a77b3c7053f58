// gdn_chunk_k64.hip -- the chunked form's kernels at compiled key width 64 (keys up to 64).
#include "gdn_chunk.hpp"

namespace gdn {
GDN_CHUNK_INSTANTIATE(64)
}  // namespace gdn
