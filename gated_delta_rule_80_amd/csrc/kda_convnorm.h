// Short causal convolution + SiLU + per-head L2 norm for one thread's tile of
// TOK consecutive tokens x 8 consecutive channels of one head.
//
// The filters are stored per channel as [H*D][K] float32, the [C, 1, K] layout of
// the released q/k/v_conv1d weights ("MaxText PR 5548", review item 2), and
// applied as a cross-correlation whose last tap multiplies the current token:
//   y[t, c] = sum_{tau=0..3} w[c, tau] * x[t - 3 + tau, c],   then SiLU.
// Inputs before t = 0 come from the carried conv state (oldest first) or zeros.
// q and k are then divided by sqrt(sum over the head's D channels of y^2 + eps).
#pragma once
#include "kda_device.h"

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

// SiLU(x) = x * sigmoid(x) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// Raw inputs of tensor `x` (one of q, k, v) for tokens t in [t_first - 3, t_first + TOK),
// channels [ch, ch + 8).  Tokens < 0 read the carried state, tokens >= T read 0.
template <int TOK, typename IO>
__device__ __forceinline__ void load_window(const IO* x, const IO* state, int tensor, int b,
                                            int T, int H, int D, int h, int ch, int t_first,
                                            float (&win)[TOK + 3][8]) {
  const size_t HD = (size_t)H * D;
#pragma unroll
  for (int m = 0; m < TOK + 3; ++m) {
    const int t = t_first - 3 + m;
    if (t >= 0 && t < T) {
      load8(x + ((size_t)b * T + t) * HD + (size_t)h * D + ch, win[m]);
    } else if (t < 0 && state != nullptr) {
      // state layout [B][3 tensors][3 taps][H*D], oldest tap first
      load8(state + (((size_t)b * 3 + tensor) * 3 + (3 + t)) * HD + (size_t)h * D + ch, win[m]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) win[m][c] = 0.f;
    }
  }
}

// conv + SiLU for TOK tokens x 8 channels of one tensor.  With conv_w == NULL
// (conv_k == 0) the raw inputs are passed through.  Outputs of tokens >= T are 0.
template <int TOK, typename IO>
__device__ __forceinline__ void conv_silu_tile(const IO* x, const IO* state, const float* conv_w,
                                               int tensor, int b, int T, int H, int D, int h,
                                               int ch, int t_first, bool active,
                                               float (&y)[TOK][8]) {
  if (!active) {
#pragma unroll
    for (int m = 0; m < TOK; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) y[m][c] = 0.f;
    return;
  }
  if (conv_w == nullptr) {
#pragma unroll
    for (int m = 0; m < TOK; ++m) {
      const int t = t_first + m;
      if (t < T) {
        load8(x + ((size_t)b * T + t) * ((size_t)H * D) + (size_t)h * D + ch, y[m]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) y[m][c] = 0.f;
      }
    }
    return;
  }
  float win[TOK + 3][8];
  load_window<TOK, IO>(x, state, tensor, b, T, H, D, h, ch, t_first, win);
  const size_t HD = (size_t)H * D;
  const float* wt = conv_w + ((size_t)tensor * HD + (size_t)h * D + ch) * 4;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(wt + 4 * c);
#pragma unroll
    for (int m = 0; m < TOK; ++m) {
      // output token t_first + m uses window rows m .. m + 3 (inputs t - 3 .. t)
      float acc = w[0] * win[m][c];
      acc = fmaf(w[1], win[m + 1][c], acc);
      acc = fmaf(w[2], win[m + 2][c], acc);
      acc = fmaf(w[3], win[m + 3][c], acc);
      y[m][c] = (t_first + m < T) ? silu_fast(acc) : 0.f;
    }
  }
}

// Full front end for q, k, v of one tile.  All lanes of a group of D/8 consecutive
// lanes (the channels of one token row) must call this together: the L2 sums are
// reduced across that group.  On return q is normalised and multiplied by
// `scale`, k normalised, v convolved; qk[m] = <q_m, k_m> of the returned values.
template <int TOK, int D, typename IO>
__device__ __forceinline__ void conv_norm_tile(const IO* q, const IO* k, const IO* v,
                                               const IO* state, const float* conv_w, int b, int T,
                                               int H, int h, int ch, int t_first, bool active,
                                               bool l2, float eps, float scale,
                                               float (&yq)[TOK][8], float (&yk)[TOK][8],
                                               float (&yv)[TOK][8], float (&qk)[TOK]) {
  conv_silu_tile<TOK, IO>(q, state, conv_w, 0, b, T, H, D, h, ch, t_first, active, yq);
  conv_silu_tile<TOK, IO>(k, state, conv_w, 1, b, T, H, D, h, ch, t_first, active, yk);
  conv_silu_tile<TOK, IO>(v, state, conv_w, 2, b, T, H, D, h, ch, t_first, active, yv);
  constexpr int G = D / 8;  // lanes sharing one token row
#pragma unroll
  for (int m = 0; m < TOK; ++m) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      sq = fmaf(yq[m][c], yq[m][c], sq);
      sk = fmaf(yk[m][c], yk[m][c], sk);
    }
    sq = group_sum<G>(sq);
    sk = group_sum<G>(sk);
    const float rq = (l2 ? 1.0f / sqrtf(sq + eps) : 1.0f) * scale;
    const float rk = l2 ? 1.0f / sqrtf(sk + eps) : 1.0f;
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      yq[m][c] *= rq;
      yk[m][c] *= rk;
      d = fmaf(yq[m][c], yk[m][c], d);
    }
    qk[m] = group_sum<G>(d);
  }
}

}  // namespace kda
