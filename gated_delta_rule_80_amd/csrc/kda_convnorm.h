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
constexpr float kLn2 = 0.6931471805599453f;

// SiLU(x) = x * sigmoid(x) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// sigmoid(x) the same way
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// softplus(x) * log2(e) = max(x, 0) log2(e) + log2(1 + 2^(-|x| log2(e))), with the
// hardware base-2 exp and log.  Where 2^(-|x| log2 e) < 2^-24 the second term
// rounds to 0 (an absolute error below 1e-7).
__device__ __forceinline__ float softplus_log2(float x) {
  const float e = __builtin_amdgcn_exp2f(-kLog2e * fabsf(x));
  return fmaf(fmaxf(x, 0.0f), kLog2e, __builtin_amdgcn_logf(1.0f + e));
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t BufRes;

// Buffer resource over `bytes` bytes from `base` (raw, no stride).  Loads through
// it are range checked: an access at or past `bytes` -- a negative 32-bit offset
// included -- returns zeros.  The third word selects 32-bit data format, as
// untyped loads need on gfx9.
// base and bytes must be the same in every lane; they are moved to scalar
// registers explicitly (a resource computed in vector registers would otherwise
// be legalised with a loop over lanes).
__device__ __forceinline__ BufRes make_buf(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  void* sbase = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(sbase, (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 8 consecutive elements kept unconverted while their load is in flight.
template <typename IO> struct Raw8;
template <> struct Raw8<__bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  // range-checked load (zeros where voff is outside the buffer); offsets in bytes
  __device__ __forceinline__ void load(BufRes r, int voff, int soff) {
    v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  // bitwise or (one of the two is all zeros)
  __device__ __forceinline__ void merge(const Raw8& o) {
    v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) | __builtin_bit_cast(u32x4, o.v));
  }
  __device__ __forceinline__ float operator[](int c) const { return (float)v[c]; }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void load(BufRes r, int voff, int soff) {
    a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0));
  }
  __device__ __forceinline__ void merge(const Raw8& o) {
    a = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, a) | __builtin_bit_cast(u32x4, o.a));
    b = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, b) | __builtin_bit_cast(u32x4, o.b));
  }
  __device__ __forceinline__ float operator[](int c) const { return c < 4 ? a[c] : b[c - 4]; }
};

// Filters of head h as [3 tensors][4 taps][D channels] float32 in LDS (taps
// outermost, so the 8 channels a thread reads for one tap are 32 contiguous
// bytes and 8 consecutive channel groups fall in distinct banks).  The global
// layout is [3][H*D][4].  load_filters issues the global loads of this
// thread's entries (call it before the other loads so those stay in flight);
// store_filters writes them transposed.  All NT threads call both; the copy is
// visible after the caller's next barrier.
template <int D, int NT>
struct FilterRegs {
  static constexpr int N = (3 * D + NT - 1) / NT;
  f32x4 w[N];
};
template <int D, int NT>
__device__ __forceinline__ void load_filters(const float* conv_w, int H, int h, int tid,
                                             FilterRegs<D, NT>& f) {
#pragma unroll
  for (int i = 0; i < FilterRegs<D, NT>::N; ++i) {
    const int e = tid + NT * i;
    const int x = e / D, c = e % D;
    if (e < 3 * D)
      f.w[i] = *reinterpret_cast<const f32x4*>(conv_w + ((size_t)x * H * D + (size_t)h * D + c) * 4);
  }
}
// `mul` scales every tap (kLog2e for front_compute's PRE mode).
template <int D, int NT>
__device__ __forceinline__ void store_filters(const FilterRegs<D, NT>& f, float* dst, int tid,
                                              float mul = 1.0f) {
#pragma unroll
  for (int i = 0; i < FilterRegs<D, NT>::N; ++i) {
    const int e = tid + NT * i;
    const int x = e / D, c = e % D;
    if (e < 3 * D) {
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) dst[(x * 4 + tau) * D + c] = f.w[i][tau] * mul;
    }
  }
}

// Raw rows of q, k, v (x = 0, 1, 2) for one thread's tile of TOK tokens from
// t_first, channels [ch, ch + 8) of head h.  The workgroup's threads together
// cover tokens [t_base, t_base + n_tok) (the same values for all of them).  Row m
// holds token t_first - 3 + m (TOK + 3 rows); with the convolution, tokens < 0
// read the carried state ([B][3 tensors][3 taps][H*D], oldest tap first).
// Without it rows 0..2 are not used (the range starts at t_base).  Rows that
// read nothing (tokens >= T, before the range, or < 0 with no state) read
// zeros: every row goes through a range-checked buffer load whose range ends at
// the sequence's last row (or the state's last tap; the check is on the
// per-lane offset, where rows before the range wrap to huge values), so all
// loads are issued unconditionally, into the same rows in both modes (a branch
// between the modes would make the compiler wait for the loads where it joins),
// with 32-bit offset arithmetic.  Needs T > 0 and
// (n_tok + 3) * H * D * sizeof(IO) < 2 GiB.
template <int TOK, typename IO>
__device__ __forceinline__ void front_load(const IO* q, const IO* k, const IO* v, const IO* state,
                                           bool conv, int b, int T, int H, int D, int h, int ch,
                                           int t_base, int n_tok, int t_first,
                                           Raw8<IO> (&win)[3][TOK + 3]) {
  constexpr int ES = (int)sizeof(IO);
  const long HD = (long)H * D;
  // rows [r0, r1) of this sequence and head: from the first row any thread reads
  // to the last one that exists
  const int r0 = conv ? (t_base - 3 > 0 ? t_base - 3 : 0) : t_base;
  const int r1 = t_base + n_tok < T ? t_base + n_tok : T;
  const unsigned bytes = (unsigned)(((long)(r1 - 1 - r0) * HD + D) * ES);
  const int row_b = (int)(HD * ES);
  const int voff = (t_first - 3 - r0) * row_b + ch * ES;  // negative rows fall out of range
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const IO* src = x == 0 ? q : (x == 1 ? k : v);
    const BufRes rx = make_buf(src + ((long)b * T + r0) * HD + (long)h * D, bytes);
#pragma unroll
    for (int m = 0; m < TOK + 3; ++m) win[x][m].load(rx, voff + m * row_b, 0);
  }
  if (conv && state != nullptr && t_base < 3) {
    // the first rows of the sequence: taps before token 0 come from the state,
    // whose 3 rows sit at "tokens" -3 .. -1 (rows past them fall out of range)
    const unsigned sbytes = (unsigned)((2 * HD + D) * ES);
    const int svoff = (t_first - 3 + 3) * row_b + ch * ES;  // token t_first - 3 is state row t_first
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const BufRes rs = make_buf(state + ((long)b * 3 + x) * 3 * HD + (long)h * D, sbytes);
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        Raw8<IO> sv;
        sv.load(rs, svoff + m * row_b, 0);
        win[x][m].merge(sv);
      }
    }
  }
}

// conv + SiLU + L2 norm of the rows front_load fetched.  `filt` is the head's
// [3][4][D] filter block written by store_filters (unused without the
// convolution).  PRE: the filters were stored times log2(e), so the convolution
// gives u = log2(e) pre and SiLU(pre) = u sigmoid(pre) / log2(e) with
// sigmoid(pre) = 1 / (1 + 2^-u): no multiply before the exponential.  The values
// returned for q and k are exact all the same (the L2 norm divides the factor
// out, its eps scaled by log2(e)^2; without the norm the factor is folded into
// the scales), but v is returned times log2(e) (multiply by kLn2) when conv.  All
// lanes of a group of D/8 consecutive lanes (the channels of one token row) must
// call this together: the L2 sums are reduced across that group.  On return q is
// normalised and multiplied by `scale`, k normalised, v convolved; qk[m] =
// <q_m, k_m> of the returned values (0 unless WANT_QK).  With MASK, tokens >= T
// and inactive lanes give zeros; without it their outputs are left as computed
// (finite).
template <int TOK, int D, typename IO, bool WANT_QK = true, bool MASK = true, bool PRE = false>
__device__ __forceinline__ void front_compute(const Raw8<IO> (&win)[3][TOK + 3], const float* filt,
                                              bool conv, int ch, int t_first,
                                              int T, bool active, bool l2, float eps, float scale,
                                              float (&yq)[TOK][8], float (&yk)[TOK][8],
                                              float (&yv)[TOK][8], float (&qk)[TOK]) {
  const bool pre = PRE && conv;                    // q, k, v come out times log2(e)
  const float unit = pre ? kLn2 : 1.0f;            // undoes that without the norm
  const float eps_n = pre ? eps * (kLog2e * kLog2e) : eps;
  float (*y[3])[8] = {yq, yk, yv};
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    if (conv) {
      float rows[TOK + 3][8];
#pragma unroll
      for (int m = 0; m < TOK + 3; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) rows[m][c] = win[x][m][c];
      float w[4][8];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(filt + (x * 4 + tau) * D + ch);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(filt + (x * 4 + tau) * D + ch + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          w[tau][c] = lo[c];
          w[tau][c + 4] = hi[c];
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int m = 0; m < TOK; ++m) {
          // output token t_first + m uses rows m .. m + 3 (inputs t - 3 .. t)
          float acc = w[0][c] * rows[m][c];
          acc = fmaf(w[1][c], rows[m + 1][c], acc);
          acc = fmaf(w[2][c], rows[m + 2][c], acc);
          acc = fmaf(w[3][c], rows[m + 3][c], acc);
          const float sv = PRE ? acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc))
                               : silu_fast(acc);
          y[x][m][c] = (!MASK || (active && t_first + m < T)) ? sv : 0.f;
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
    const float rq = (l2 ? __builtin_amdgcn_rsqf(sq + eps_n) : unit) * scale;
    const float rk = l2 ? __builtin_amdgcn_rsqf(sk + eps_n) : unit;
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
