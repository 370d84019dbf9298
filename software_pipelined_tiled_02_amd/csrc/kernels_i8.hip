// kernels_i8.hip -- pipelined GEMM kernel instances for i8 inputs.
#include "instances.h"

namespace pg {

const KernelEntry* kernels_i8(int* count) {
    static KernelEntry table[kInstancesPerDtype];
    static const int n = fill_instances<DT_I8>(table);
    *count = n;
    return table;
}

}  // namespace pg
