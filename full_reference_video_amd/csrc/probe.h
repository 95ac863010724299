// probe.h — the fp32 VALU probe of probe.hip (library-private).
#pragma once

#include <hip/hip_runtime.h>

#include "vqm_kernels.h"

namespace vqm {

// `blocks` workgroups of 256 threads, each thread running 16 independent
// FMA chains for `iters` steps; out receives 256 blocks floats.
// valu_probe_fmas gives the lane FMAs of one launch.
long long valu_probe_fmas(int blocks, int iters);
hipError_t launch_valu_probe(float *out, int blocks, int iters, hipStream_t stream, const KernelTimer &timer);

}  // namespace vqm
