// Batched / prefill regime (more than 8 tokens): the union-of-active-channels
// path on bf16 MFMA. Not built yet: the dispatcher reports it as unsupported.
#include "sffn_internal.h"

namespace sffn {

hipError_t launch_batched(sffn_ctx &, const FwdArgs &) { return hipErrorNotSupported; }

}  // namespace sffn
