// stk_prof.hpp -- optional HIP-event timing of individual kernels.
//
// When a kernel's bit is enabled (soft_topk_profile_begin), its launchers
// record one event pair on the launch stream around each launch; the pairs
// are resolved by soft_topk_profile_end.  Disabled bits cost one relaxed
// atomic load per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace stk {

enum KernelId : int {
    kKSample = 0,   // the diagnostic sampler
    kKFilter,
    kKSelect,
    kKPass1,
    kKBandHist,
    kKBandScatter,
    kKBucketAgg,
    kKSolve,
    kKRadixUp,
    kKRadixDown,
    kKRadixScan,
    kKTileAgg,
    kKEmit,
    kKEmitFinal,
    kKVjpReduce,
    kKVjpApply,
    kKReset,
    kKRowsForward,
    kKRowsBackward,
    kKCurveScan,
    kKCurve,
    kKIterate,      // partition refinement (every kernel of it)
    kKernelCount
};

const char* kernel_name(int id);
void prof_before(int id, hipStream_t stream);
void prof_after(int id, hipStream_t stream);

}  // namespace stk

// Launch with optional timing: STK_LAUNCH(id, stream, kernel, grid, block, shmem, stream, args...)
#define STK_LAUNCH(id, strm, ...)            \
    do {                                     \
        ::stk::prof_before((id), (strm));    \
        hipLaunchKernelGGL(__VA_ARGS__);     \
        ::stk::prof_after((id), (strm));     \
    } while (0)
