// Decode attention kernels for header-free records (one fixed quantizer per head)
// of the formats of the 64-bit per-vector budget.
#include "attend_spec.h"

namespace kvtc {
KVTC_DEFINE_SPEC_CLASS(4)
}  // namespace kvtc
