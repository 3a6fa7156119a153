// Optional per-kernel timing with HIP events recorded on the launch stream
// around every kernel of the library. Off by default; when off the hooks cost
// one relaxed atomic load per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace smoe {

enum KernelId {
    kKRouteLogits = 0,
    kKRouteTopk,
    kKMapHist,
    kKMapRowscan,
    kKMapAssign,
    kKMapEmpty,
    kKTileTable,
    kKAccZero,
    kKGateUp,
    kKDown,
    kKFinalize,
    kKCombine,
    kKPlGemm,
    kKPlDxGemm,
    kKPlWgrad,
    kKPlPrep,
    kKPlFinalize,
    kKBwdRecompute,
    kKBwdDh,
    kKBwdPrep,
    kKBwdWgrad,
    kKBwdDx,
    kKMapSmall,
    kNumKernelIds
};

const char *kernel_name(int id);
void prof_begin(hipStream_t stream, int id);
void prof_end(hipStream_t stream, int id);

}  // namespace smoe
