// ring_kernel_f32.hip -- float32 instantiations of the ring AllReduce kernel:
// every (operator, protocol) pair.
#include "ring_kernel.h"

namespace rar {
const void* get_ring_kernel_f32(int proto, int red) { return ring_kernel_table<TyF32>(proto, red); }
}  // namespace rar
