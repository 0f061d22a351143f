// Single-query-row decode kernel (placeholder until the streaming kernel lands).
#include "common.h"
#include "kernels.h"

namespace attn {
int decode_keys_per_tile() { return 64; }
int decode_max_rows() { return 0; }
hipError_t launch_fwd_decode(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
