// stream_read.h -- the streaming-read yardstick launch (mr_debug_stream_read).
// Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mr {

// Plain streaming read of nbytes (a multiple of 16, 16-byte aligned): block b
// of at most kStreamReadMaxBlocks stores the XOR of the words it read in
// out[b]; the XOR of out[0 .. kStreamReadMaxBlocks) is the XOR of every word
// when out starts zeroed.
constexpr int kStreamReadMaxBlocks = 4096;
hipError_t launch_stream_read(const void *src, size_t nbytes, uint32_t *out, hipStream_t stream);

}  // namespace mr
