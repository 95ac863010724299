// probe.h — the inspection kernels of probe.hip (library-private).
#pragma once

#include <hip/hip_runtime.h>

#include "vqm_kernels.h"

namespace vqm {

// A streaming read of bytes / 16 16-byte vectors of buf (non-temporal loads,
// one workgroup of 256 threads per 64 KiB); sink receives one word per
// workgroup (read_probe_blocks of them).
long long read_probe_blocks(long long bytes);
hipError_t launch_read_probe(const void *buf, long long bytes, uint32_t *sink, hipStream_t stream,
                             const KernelTimer &timer);

// The fp32 VALU probe: `blocks` workgroups of 256 threads, each thread
// running 16 independent FMA chains for `iters` steps; out receives
// 256 blocks floats.  valu_probe_fmas gives the lane FMAs of one launch.
long long valu_probe_fmas(int blocks, int iters);
hipError_t launch_valu_probe(float *out, int blocks, int iters, hipStream_t stream, const KernelTimer &timer);

}  // namespace vqm
