// kernels_f32.hip -- pipelined GEMM kernel instances for f32 inputs.
#include "instances.h"

namespace pg {

const KernelEntry* kernels_f32(int* count) {
    static KernelEntry table[kInstancesPerDtype];
    static const int n = fill_instances<DT_F32>(table);
    *count = n;
    return table;
}

}  // namespace pg
