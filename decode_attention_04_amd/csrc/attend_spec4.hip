// Decode attention kernels for the mixed layout of full-rank 2-bit and rank-16
// 6-bit heads.
#include "attend_spec.h"

namespace kvtc {
KVTC_DEFINE_SPEC_CLASS(4)
}  // namespace kvtc
