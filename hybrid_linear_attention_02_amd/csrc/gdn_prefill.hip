#include <hip/hip_runtime.h>
#include "gdn_internal.h"
namespace gdn {
int launch_prefill(const gdn_pool*, const gdn_prefill_args*, const PrefillPlan&, void*, void*) {
    return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: not built yet");
}
}
