// The measured int8 MFMA ceiling (k_ceiling.hip), internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmf {

// `blocks` workgroups of four waves, each wave `iters` rounds of four
// independent 32x32x32 int8 MFMAs; one sink word per workgroup;
// mfma_loop_ops counts the operations of such a launch.
int mfma_ceiling_blocks(int cus);
hipError_t launch_mfma_loop(int64_t iters, int blocks, uint32_t *sink, hipStream_t st);
int64_t mfma_loop_ops(int64_t iters, int blocks);

}  // namespace mmf
