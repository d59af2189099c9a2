// Decode attention kernels for the record formats of the 128-bit budget class.
#include "attend_spec.h"

namespace kvtc {
KVTC_DEFINE_SPEC_CLASS(1)
}  // namespace kvtc
