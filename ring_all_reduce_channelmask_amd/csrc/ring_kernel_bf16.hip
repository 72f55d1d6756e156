// ring_kernel_bf16.hip -- bfloat16 instantiations of the ring AllReduce kernel:
// every (operator, protocol) pair.
#include "ring_kernel.h"

namespace rar {
const void* get_ring_kernel_bf16(int proto, int red) { return ring_kernel_table<TyBF16>(proto, red); }
}  // namespace rar
