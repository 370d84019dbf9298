// instances.h -- the kernel instances one translation unit compiles for one
// input type: both layouts at every tile class, each at stages 1-4 and both
// load variants, plus the register-staged variant's instances for a K that
// is not a multiple of 16 bytes.
#ifndef PIPEGEMM_INSTANCES_H
#define PIPEGEMM_INSTANCES_H

#include "gemm_kernel.h"

namespace pg {

template <int DT, int LAYOUT, int TC, int S, int V>
inline KernelEntry entry() {
    return KernelEntry{DT, LAYOUT, TC, S, V, (const void*)&pipegemm_kernel<DT, LAYOUT, TC, S, V>};
}

template <int DT, int LAYOUT, int TC>
inline void add_tile(KernelEntry* t, int& n) {
    t[n++] = entry<DT, LAYOUT, TC, 1, VAR_REG>();
    t[n++] = entry<DT, LAYOUT, TC, 2, VAR_REG>();
    t[n++] = entry<DT, LAYOUT, TC, 3, VAR_REG>();
    t[n++] = entry<DT, LAYOUT, TC, 4, VAR_REG>();
    t[n++] = entry<DT, LAYOUT, TC, 1, VAR_DIRECT>();
    t[n++] = entry<DT, LAYOUT, TC, 2, VAR_DIRECT>();
    t[n++] = entry<DT, LAYOUT, TC, 3, VAR_DIRECT>();
    t[n++] = entry<DT, LAYOUT, TC, 4, VAR_DIRECT>();
    t[n++] = entry<DT, LAYOUT, TC, 1, VAR_REG_KTAIL>();
    t[n++] = entry<DT, LAYOUT, TC, 2, VAR_REG_KTAIL>();
    t[n++] = entry<DT, LAYOUT, TC, 3, VAR_REG_KTAIL>();
    t[n++] = entry<DT, LAYOUT, TC, 4, VAR_REG_KTAIL>();
}

constexpr int kInstancesPerDtype = 8 * 12;

template <int DT>
inline int fill_instances(KernelEntry* t) {
    int n = 0;
    add_tile<DT, LAYOUT_RC, TILE_L>(t, n);
    add_tile<DT, LAYOUT_RC, TILE_W>(t, n);
    add_tile<DT, LAYOUT_RC, TILE_M>(t, n);
    add_tile<DT, LAYOUT_RC, TILE_T>(t, n);
    add_tile<DT, LAYOUT_RR, TILE_L>(t, n);
    add_tile<DT, LAYOUT_RR, TILE_W>(t, n);
    add_tile<DT, LAYOUT_RR, TILE_M>(t, n);
    add_tile<DT, LAYOUT_RR, TILE_T>(t, n);
    return n;
}

}  // namespace pg

#endif
