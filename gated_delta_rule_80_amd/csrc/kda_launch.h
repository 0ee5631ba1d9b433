// Kernel launchers (defined next to their kernels, called by the host runtime).
#pragma once
#include <hip/hip_runtime.h>

#include "kda_layout.h"

namespace kda {

hipError_t launch_prep(const PrepParams& p, int D, int C, bool fp32, hipStream_t st);
hipError_t launch_prep_exact(const PrepParams& p, int D, int C, bool fp32, unsigned grid,
                             hipStream_t st);
hipError_t launch_state(const StateParams& p, int D, int C, bool fp32, int vb, int threads, bool gn,
                        hipStream_t st);
hipError_t launch_out_stage(const OutStageParams& p, int D, bool fp32, hipStream_t st);
hipError_t launch_conv_norm(const ConvNormParams& p, int D, bool fp32, hipStream_t st);
hipError_t launch_conv_tail(const TailParams& p, bool fp32, hipStream_t st);
hipError_t launch_seq_index(const IndexParams& p, hipStream_t st);
hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t st);
hipError_t launch_backward(const BwdLaunch& L, int D, int C, bool fp32, hipStream_t st);
size_t bwd_front_blocks(int T, int D);
hipError_t launch_decode(const DecodeParams& p, int D, bool fp32, hipStream_t st);

}  // namespace kda
