// gdn_chunked.hip -- chunked prefill (placeholder until the kernel lands).
#include "gdn_internal.hpp"

namespace gdn {

size_t chunked_workspace_bytes(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d,
                               int chunk)
{
    (void)n; (void)t; (void)h_qk; (void)h_v; (void)d; (void)chunk;
    return 0;
}

hipError_t launch_chunked(const Call& c, int chunk)
{
    (void)c; (void)chunk;
    return hipErrorNotSupported;
}

}  // namespace gdn
