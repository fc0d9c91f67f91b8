// sa_stream_d128.h -- launcher of the software-pipelined streaming forward
// for heads of width 128 on the history axis (sa_stream_d128.hip).
#pragma once

#include "sa_internal.h"

namespace sa {

// Block shape for dh = 128: one head and 256 prototypes per block (8 waves),
// m / 256 blocks per head; false unless m is a multiple of 256.
bool stream_d128_config(int m, int H, StreamConfig* cfg);

// History axis (a.norm == 0), a.dh == 128: writes the segments' partial
// statistics (M, Z and the lane-major weighted sums) for sa_merge_kernel.
hipError_t launch_stream_d128(const FwdArgs& a, const StreamConfig& cfg, hipStream_t s);

}  // namespace sa
