// Kernel launchers (defined next to their kernels, called by the host runtime).
#pragma once
#include <hip/hip_runtime.h>

#include "kda.h"
#include "kda_layout.h"

namespace kda {

hipError_t launch_prep(const PrepParams& p, int D, int C, bool fp32, hipStream_t st);
hipError_t launch_prep_exact(const PrepParams& p, int D, int C, bool fp32, unsigned grid,
                             hipStream_t st);
hipError_t launch_state(const StateParams& p, int D, int C, bool fp32, int vb, int threads, bool gn,
                        hipStream_t st);
// split state walk: the segments' maps, then their start states (SplitParams)
hipError_t launch_split_maps(const SplitParams& p, int D, int C, bool fp32, int vb, int threads,
                             hipStream_t st);
hipError_t launch_split_combine(const SplitParams& p, int D, hipStream_t st);
// the state map of a whole call (SplitParams.whole): segment maps, then their
// composition into M_out, N_out; and M = I, N = 0 for n matrices of D x D
hipError_t launch_state_map(const SplitParams& p, int D, int C, bool fp32, int vb, int threads,
                            hipStream_t st);
hipError_t launch_state_map_identity(float* M, float* N, size_t n, int D, hipStream_t st);
hipError_t launch_out_stage(const OutStageParams& p, int D, bool fp32, hipStream_t st);
hipError_t launch_conv_norm(const ConvNormParams& p, int D, bool fp32, hipStream_t st);
hipError_t launch_conv_tail(const TailParams& p, bool fp32, hipStream_t st);
hipError_t launch_seq_index(const IndexParams& p, hipStream_t st);
hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t st);
hipError_t launch_backward(const BwdLaunch& L, int D, int C, bool fp32, hipStream_t st);
size_t bwd_front_blocks(int T, int D);
int bwd_front_tokens(int D);  // tokens per front-end workgroup of the backward
// the optional stages' backward; dw, dA_log, ddt_bias may be NULL (not written)
hipError_t launch_bwd_out_stage(const BwdOutParams& p, float* dw, int D, bool fp32, hipStream_t st);
hipError_t launch_bwd_act(const BwdActParams& p, float* dA_log, float* ddt_bias, int D, bool fp32,
                          hipStream_t st);
// packed batches: zero the conv-history gradient of the empty sequences
hipError_t launch_bwd_empty_history(float* dconv_state, const int* bounds, int n_seqs, long per_seq,
                                    hipStream_t st);
int bwd_out_groups(long rows, int D);   // workgroups (= partials) of the two
int bwd_act_groups(long tokens, int D);
hipError_t launch_decode(const DecodeParams& p, int D, bool fp32, hipStream_t st);

// The whole prefill (arguments already validated) in a workspace of `bytes`:
// time slices when the whole-sequence workspace does not fit (B equal-length
// sequences only; KDA_ERR_SCRATCH otherwise, or when one chunk per (sequence,
// head) does not fit).  Defined with the host runtime.
kda_status prefill_in_workspace(const kda_prefill_args* a, void* ws, size_t bytes, hipStream_t st);

}  // namespace kda
