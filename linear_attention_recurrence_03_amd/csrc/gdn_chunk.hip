// gdn_chunk.hip -- chunked form of the gated delta rule (placeholder).
#include "gdn_internal.h"

namespace gdn {

size_t chunk_workspace_bytes(int, int64_t, int64_t, int64_t, int)
{
    return 0;
}

hipError_t launch_chunked(const Problem &p, void *, hipStream_t stream)
{
    return launch_recurrent(p, stream);
}

}  // namespace gdn
