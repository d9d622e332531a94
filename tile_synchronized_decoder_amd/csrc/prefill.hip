// The prefill kernels (bf16 models): the prefill interpreter and one kernel per
// prefill op, compiled once.
#define MK_PREFILL_UNIT 1
#include "kernels.h"

namespace mkd {
Table table_prefill() { return {PrefillLaunch::prep, PrefillLaunch::mega, nullptr, PrefillLaunch::kpo, nullptr, nullptr, nullptr}; }
}  // namespace mkd
