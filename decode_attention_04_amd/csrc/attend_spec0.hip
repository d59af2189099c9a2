// Decode attention kernels for the record formats of the 64-bit budget class.
#include "attend_spec.h"

namespace kvtc {
KVTC_DEFINE_SPEC_CLASS(0)
}  // namespace kvtc
