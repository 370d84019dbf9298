// kernels_bf16.hip -- pipelined GEMM kernel instances for bf16 inputs.
#include "instances.h"

namespace pg {

const KernelEntry* kernels_bf16(int* count) {
    static KernelEntry table[kInstancesPerDtype];
    static const int n = fill_instances<DT_BF16>(table);
    *count = n;
    return table;
}

}  // namespace pg
