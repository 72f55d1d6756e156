// ring_kernel_i32.hip -- int32 instantiations of the ring AllReduce kernel:
// every (operator, protocol) pair.
#include "ring_kernel.h"

namespace rar {
const void* get_ring_kernel_i32(int proto, int red) { return ring_kernel_table<TyI32>(proto, red); }
}  // namespace rar
