// Decode attention kernels for a frozen cross-head allocation of the LLaMA-shaped
// layer (odd bit widths beside power-of-two ones).
#include "attend_spec.h"

namespace kvtc {
KVTC_DEFINE_SPEC_CLASS(5)
}  // namespace kvtc
