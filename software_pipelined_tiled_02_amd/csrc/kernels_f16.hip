// kernels_f16.hip -- pipelined GEMM kernel instances for f16 inputs.
#include "instances.h"

namespace pg {

const KernelEntry* kernels_f16(int* count) {
    static KernelEntry table[kInstancesPerDtype];
    static const int n = fill_instances<DT_F16>(table);
    *count = n;
    return table;
}

}  // namespace pg
