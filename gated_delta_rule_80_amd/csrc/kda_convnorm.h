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

// 8 consecutive elements kept unconverted while their load is in flight.
template <typename IO> struct Raw8;
template <> struct Raw8<__bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ float operator[](int c) const { return (float)v[c]; }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int c) const { return c < 4 ? a[c] : b[c - 4]; }
};

// Filters of head h, [3 tensors][D channels][4 taps] float32 (3*D entries of 16
// bytes), copied to LDS `dst` with the direct global-to-LDS path.  Called by all
// NT threads of the block; the copy is complete after the caller's next
// s_waitcnt vmcnt(0) and barrier.
template <int D, int NT>
__device__ __forceinline__ void stage_filters(const float* conv_w, int H, int h, float* dst, int tid) {
  constexpr int N = 3 * D;
  const int lane = tid & 63;
  for (int base = tid - lane; base < N; base += NT) {  // wave-uniform
    const int e = base + lane;
    if (e < N) {
      const int x = e / D, c = e % D;
      __builtin_amdgcn_global_load_lds(
          (const glb_void_t*)(conv_w + ((size_t)x * H * D + (size_t)h * D + c) * 4),
          (lds_void_t*)(dst + 4 * base), 16, 0, 0);
    }
  }
}

// 32 zero bytes: the load source of every row that reads nothing.  A plain
// global variable (never written), so a choice between it and an input row is
// still a global address and the loads stay global loads.
static __device__ __attribute__((aligned(16))) float kZeroRow[8];

template <typename IO>
__device__ __forceinline__ const IO* zero_row() {
  return reinterpret_cast<const IO*>(kZeroRow);
}

// Raw rows of q, k, v (x = 0, 1, 2) for one thread's tile of TOK tokens from
// t_first, channels [ch, ch + 8) of head h.  With the convolution, row m holds
// token t_first - 3 + m (TOK + 3 rows); tokens < 0 read the carried state
// ([B][3 tensors][3 taps][H*D], oldest tap first).  Without it, row 3 + m holds
// token t_first + m.  Rows that read nothing (tokens >= T, or < 0 with no state)
// read zeros, so every load is issued unconditionally and all of them are in
// flight together.
template <int TOK, typename IO>
__device__ __forceinline__ void front_load(const IO* q, const IO* k, const IO* v, const IO* state,
                                           bool conv, int b, int T, int H, int D, int h, int ch,
                                           int t_first, Raw8<IO> (&win)[3][TOK + 3]) {
  const size_t HD = (size_t)H * D;
  const size_t row0 = (size_t)b * T * HD + (size_t)h * D + ch;
  const IO* src[3] = {q, k, v};
  if (conv) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const IO* srow = state == nullptr ? nullptr
                                        : state + ((size_t)b * 3 + x) * 3 * HD + (size_t)h * D + ch;
#pragma unroll
      for (int m = 0; m < TOK + 3; ++m) {
        const int t = t_first - 3 + m;
        const IO* ptr = zero_row<IO>();
        if (t >= 0 && t < T) ptr = src[x] + row0 + (size_t)t * HD;
        else if (t < 0 && srow != nullptr) ptr = srow + (size_t)(3 + t) * HD;
        win[x][m].load(ptr);
      }
    }
  } else {
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int m = 0; m < TOK; ++m) {
        const int t = t_first + m;
        win[x][3 + m].load(t < T ? src[x] + row0 + (size_t)t * HD : zero_row<IO>());
      }
  }
}

// conv + SiLU + L2 norm of the rows front_load fetched.  `filt` is the head's
// [3][D][4] filter block (LDS or global; unused without the convolution).  All
// lanes of a group of D/8 consecutive lanes (the channels of one token row) must
// call this together: the L2 sums are reduced across that group.  On return q is
// normalised and multiplied by `scale`, k normalised, v convolved; qk[m] =
// <q_m, k_m> of the returned values (0 unless WANT_QK).  With MASK, tokens >= T
// and inactive lanes give zeros; without it their outputs are left as computed
// (finite).
template <int TOK, int D, typename IO, bool WANT_QK = true, bool MASK = true>
__device__ __forceinline__ void front_compute(const Raw8<IO> (&win)[3][TOK + 3], const float* filt,
                                              bool conv, int ch, int t_first,
                                              int T, bool active, bool l2, float eps, float scale,
                                              float (&yq)[TOK][8], float (&yk)[TOK][8],
                                              float (&yv)[TOK][8], float (&qk)[TOK]) {
  float (*y[3])[8] = {yq, yk, yv};
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    if (conv) {
      float rows[TOK + 3][8];
#pragma unroll
      for (int m = 0; m < TOK + 3; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) rows[m][c] = win[x][m][c];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(filt + ((size_t)x * D + ch + c) * 4);
#pragma unroll
        for (int m = 0; m < TOK; ++m) {
          // output token t_first + m uses rows m .. m + 3 (inputs t - 3 .. t)
          float acc = w[0] * rows[m][c];
          acc = fmaf(w[1], rows[m + 1][c], acc);
          acc = fmaf(w[2], rows[m + 2][c], acc);
          acc = fmaf(w[3], rows[m + 3][c], acc);
          y[x][m][c] = (!MASK || (active && t_first + m < T)) ? silu_fast(acc) : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < TOK; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          y[x][m][c] = (!MASK || (active && t_first + m < T)) ? win[x][3 + m][c] : 0.f;
    }
  }
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
    const float rq = (l2 ? __builtin_amdgcn_rsqf(sq + eps) : 1.0f) * scale;
    const float rk = l2 ? __builtin_amdgcn_rsqf(sk + eps) : 1.0f;
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      yq[m][c] *= rq;
      yk[m][c] *= rk;
      d = fmaf(yq[m][c], yk[m][c], d);
    }
    qk[m] = WANT_QK ? group_sum<G>(d) : 0.f;
  }
}

}  // namespace kda
