// Decode kernels with K codec 2 (see decode_impl.h); one file per K codec so
// the 25 codec pairs x 3 row layouts compile in parallel.
#include "decode_impl.h"

namespace vit {
VIT_DECODE_FOR_K(2)
}  // namespace vit
