// scratch.hip -- the library-held scratch of attn_decode_fwd_noalloc.
//
// One array per GPU, in the code object's zero-initialised data: the split
// partials and arrival counters of calls whose callers cannot allocate.  Host
// code must not pass the array's name to a kernel (on the host it is only a
// stand-in for the registered variable); it asks the runtime for the array's
// device address once per device and uses that address.
#include "internal.h"

namespace skv {

static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

hipError_t scratch_device_address(void** ptr) {
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch));
}

}  // namespace skv
