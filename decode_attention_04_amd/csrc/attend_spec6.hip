// Decode attention kernels for vector-quantized records: coordinate pairs with
// per-pair codebooks held in LDS, and a per-token scale word.
#include "attend_spec.h"

namespace kvtc {
KVTC_DEFINE_SPEC_CLASS(6)
}  // namespace kvtc
