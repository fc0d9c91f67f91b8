// sa_proto.h -- launcher of the one-pass prototype-axis kernel
// (sa_proto_stream.hip).
#pragma once

#include "sa_internal.h"

namespace sa {

// Whether the one-pass kernel serves a streaming configuration: every block
// must hold all m prototypes of its heads (NH * m / 32 == NW), which is the
// case for every dh = 32 / 64 shape of stream_config.
bool proto_one_pass(const StreamConfig& cfg, int dh);

// Prototype axis in one pass over K and V (a.norm == 1, shared prototypes):
// writes the segments' weighted sums to a.part.acc for sa_merge_kernel, and,
// when lse_out is not null, the natural-log row normaliser lse_out[row * H + h]
// of every row the segments visit (valid rows: the value; masked rows: -inf).
// Rows outside every user are not visited: fill_f32 sets them first.
hipError_t launch_proto_stream(const FwdArgs& a, float* lse_out, const StreamConfig& cfg, hipStream_t s);

// lse_out[0 .. n) = -inf, or NaN when the offsets check rejected the call
// (status may be null).
hipError_t launch_fill_lse(float* lse_out, int64_t n, const int32_t* status, hipStream_t s);

}  // namespace sa
