// prefill.hip — chunked causal prefill over paged K/V (placeholder: no kernel yet).
#include "device_common.h"
#include "launch.h"

namespace pa {

int launch_prefill(const PrefillParams &, void *) { return -1; }

}  // namespace pa
