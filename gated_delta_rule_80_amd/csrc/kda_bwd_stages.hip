// Backward of the optional stages around the mixer.
//
// Output stage, per (token, head) row of D values: from the mixer's output x
// (before the stage), the gate pre-activation z and the gradient dy of the
// stage's output, with r = 1 / sqrt(mean_c x_c^2 + eps), n = x r, a = n w (a = x
// without the norm), s = sigmoid(z) and y = a s (y = a without the gate):
//   dz = dy a s (1 - s),   da = dy s,   dw += da n,   dn = da w,
//   dx = r (dn - n mean_c(dn n))      (the norm's Jacobian applied to dn).
// Activations: with g = -exp(A_log[h]) softplus(f + dt_bias[c]) and beta =
// sigmoid(b), the gradients of the raw projections are
//   df = dg (-exp(A_log[h])) sigmoid(f + dt_bias[c]),   db = dbeta beta (1 - beta),
// and the parameters' dA_log[h] = sum dg g, ddt_bias[c] = sum df over tokens.
//
// Parameter gradients are sums over tokens: each workgroup sums a fixed set of
// rows in a fixed order into a partial, and kda_bwd_sum_kernel adds the partials
// in a fixed order, so every call gives the same bits.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

// Whether token t belongs to a sequence (packed batches: the clamped bounds are
// non-decreasing, so the sequences cover [bounds[0], bounds[n_seqs]) exactly).
__device__ __forceinline__ bool token_in_seqs(long t, const SeqTables& sq) {
  return sq.bounds == nullptr || (t >= sq.bounds[0] && t < sq.bounds[sq.n_seqs]);
}

// One pass over the rows: D / 8 threads per row, each with 8 consecutive
// channels; a workgroup takes RPW rows at a time and strides over the rows
// with the grid.
template <int D, typename IO>
__global__ __launch_bounds__(256) void kda_bwd_out_kernel(BwdOutParams p) {
  constexpr int G = D / 8;      // threads per row
  constexpr int RPW = 256 / G;  // rows per workgroup and pass
  const int tid = threadIdx.x, j = tid % G, rr = tid / G;
  const bool norm = p.w != nullptr, gate = p.z != nullptr;
  float w[8], dwacc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    w[c] = 1.f;
    dwacc[c] = 0.f;
  }
  if (norm) load8(p.w + 8 * j, w);
  // every thread runs the same number of passes (the group sums need the whole row)
  for (long base = (long)blockIdx.x * RPW; base < p.rows; base += (long)gridDim.x * RPW) {
    const long row = base + rr;
    const bool ok = row < p.rows && token_in_seqs(row / p.H, p.seqs);
    float x[8], z[8], dy[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = z[c] = dy[c] = 0.f;
    if (ok) {
      load8(static_cast<const IO*>(p.x) + row * D + 8 * j, x);
      load8(static_cast<const IO*>(p.dy) + row * D + 8 * j, dy);
      if (gate) load8(static_cast<const IO*>(p.z) + row * D + 8 * j, z);
    }
    float r = 1.f;
    if (norm) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(x[c], x[c], ss);
      ss = group_sum<G>(ss);
      r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
    }
    float n[8], da[8], dz[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      n[c] = x[c] * r;
      const float a = n[c] * w[c];
      if (gate) {
        const float s = sigmoid(z[c]);
        dz[c] = dy[c] * a * s * (1.f - s);
        da[c] = dy[c] * s;
      } else {
        dz[c] = 0.f;
        da[c] = dy[c];
      }
    }
    float dx[8];
    if (norm) {
      float t = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        dwacc[c] = fmaf(da[c], n[c], dwacc[c]);  // zero for rows past the end
        da[c] *= w[c];                            // dn
        t = fmaf(da[c], n[c], t);
      }
      t = group_sum<G>(t) * (1.0f / D);
#pragma unroll
      for (int c = 0; c < 8; ++c) dx[c] = r * (da[c] - n[c] * t);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) dx[c] = da[c];
    }
    if (ok) {
      store8(static_cast<IO*>(p.dx) + row * D + 8 * j, dx);
      if (gate && p.dz != nullptr) store8(p.dz + row * D + 8 * j, dz);
    }
  }
  if (norm && p.dw_part != nullptr) {
    // the workgroup's partial of dw: its RPW row slots summed in order
    __shared__ float sdw[RPW][D];
#pragma unroll
    for (int c = 0; c < 8; ++c) sdw[rr][8 * j + c] = dwacc[c];
    __syncthreads();
    for (int c = tid; c < D; c += 256) {
      float acc = 0.f;
      for (int q = 0; q < RPW; ++q) acc += sdw[q][c];
      p.dw_part[(size_t)blockIdx.x * D + c] = acc;
    }
  }
}

// Activations: workgroup (blockIdx.x, h) strides over the tokens of head h, TPW
// tokens at a time, D / 8 threads per token.
template <int D, typename IO>
__global__ __launch_bounds__(256) void kda_bwd_act_kernel(BwdActParams p) {
  constexpr int G = D / 8;
  constexpr int TPW = 256 / G;
  const int tid = threadIdx.x, j = tid % G, tt = tid / G;
  const int h = blockIdx.y, H = p.H;
  const bool act = p.f != nullptr;
  float bias[8], ddt[8], dA = 0.f;
  float neg_rate = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) bias[c] = ddt[c] = 0.f;
  if (act) {
    load8(p.dt_bias + (size_t)h * D + 8 * j, bias);
    neg_rate = -__expf(p.A_log[h]);
  }
  for (long base = (long)blockIdx.x * TPW; base < p.tokens; base += (long)gridDim.x * TPW) {
    const long t = base + tt;
    if (t >= p.tokens || !token_in_seqs(t, p.seqs)) continue;  // no cross-lane work in this loop
    const size_t row = ((size_t)t * H + h) * D + 8 * j;
    if (act) {
      float f[8], dg[8];
      load8(static_cast<const IO*>(p.f) + row, f);
      load8(p.dg + row, dg);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float zc = f[c] + bias[c];
        dA = fmaf(dg[c], gate_decay(f[c], bias[c], neg_rate), dA);
        dg[c] *= neg_rate * sigmoid(zc);
        ddt[c] += dg[c];
      }
      store8(p.dg + row, dg);
    }
    if (p.beta != nullptr && j == 0) {
      const size_t o = (size_t)t * H + h;
      const float b = p.beta[o];
      p.dbeta[o] *= b * (1.f - b);
    }
  }
  if (!act) return;
  __shared__ float sdd[TPW][D];
  __shared__ float sda[256];
#pragma unroll
  for (int c = 0; c < 8; ++c) sdd[tt][8 * j + c] = ddt[c];
  sda[tid] = dA;
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    float acc = 0.f;
    for (int q = 0; q < TPW; ++q) acc += sdd[q][c];
    p.ddt_part[(size_t)blockIdx.x * H * D + (size_t)h * D + c] = acc;
  }
  if (tid == 0) {
    float acc = 0.f;
    for (int q = 0; q < 256; ++q) acc += sda[q];
    p.dA_part[(size_t)blockIdx.x * H + h] = acc;
  }
}

// Packed batches: the conv-history gradient of every empty sequence is zero (no
// front-end workgroup covers such a sequence); the others' entries are left alone.
__global__ __launch_bounds__(256) void kda_bwd_empty_history_kernel(float* dconv_state, const int* bounds,
                                                                    int n_seqs, long per_seq) {
  const long total = (long)n_seqs * per_seq;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    const long s = i / per_seq;
    if (bounds[s + 1] == bounds[s]) dconv_state[i] = 0.f;
  }
}

hipError_t launch_bwd_empty_history(float* dconv_state, const int* bounds, int n_seqs, long per_seq,
                                    hipStream_t st) {
  if (dconv_state == nullptr || n_seqs <= 0 || per_seq <= 0) return hipSuccess;
  const long total = (long)n_seqs * per_seq;
  const long want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(kda_bwd_empty_history_kernel, dim3(grid), dim3(256), 0, st, dconv_state, bounds, n_seqs,
                     per_seq);
  return hipGetLastError();
}

// out[i] = sum over q = 0 .. nparts - 1 of part[q * n + i], one wave per output:
// lane l adds parts l, l + 64, ... in order, then a fixed butterfly over the lanes.
__global__ __launch_bounds__(256) void kda_bwd_sum_kernel(const float* part, float* out, size_t n,
                                                          int nparts) {
  const size_t i = (size_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  float acc = 0.f;
  if (i < n)
    for (int q = lane; q < nparts; q += 64) acc += part[(size_t)q * n + i];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (i < n && lane == 0) out[i] = acc;
}

static hipError_t launch_sum(const float* part, float* out, size_t n, int nparts, hipStream_t st) {
  if (out == nullptr || n == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_bwd_sum_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, part, out, n,
                     nparts);
  return hipGetLastError();
}

int bwd_out_groups(long rows, int D) {
  const long rpw = 256 / (D / 8);
  const long need = (rows + rpw - 1) / rpw;
  return (int)(need < kBwdStageGroups ? (need > 0 ? need : 1) : kBwdStageGroups);
}

int bwd_act_groups(long tokens, int D) {
  const long tpw = 256 / (D / 8);
  const long need = (tokens + tpw - 1) / tpw;
  const long cap = kBwdStageGroups / 8;
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

template <int D, typename IO>
static hipError_t launch_out_t(const BwdOutParams& p, float* dw, hipStream_t st) {
  const int ng = bwd_out_groups(p.rows, D);
  hipLaunchKernelGGL((kda_bwd_out_kernel<D, IO>), dim3((unsigned)ng), dim3(256), 0, st, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return p.w != nullptr ? launch_sum(p.dw_part, dw, D, ng, st) : hipSuccess;
}

hipError_t launch_bwd_out_stage(const BwdOutParams& p, float* dw, int D, bool fp32, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  switch (D) {
    case 16: return fp32 ? launch_out_t<16, float>(p, dw, st) : launch_out_t<16, __bf16>(p, dw, st);
    case 32: return fp32 ? launch_out_t<32, float>(p, dw, st) : launch_out_t<32, __bf16>(p, dw, st);
    case 64: return fp32 ? launch_out_t<64, float>(p, dw, st) : launch_out_t<64, __bf16>(p, dw, st);
    case 128: return fp32 ? launch_out_t<128, float>(p, dw, st) : launch_out_t<128, __bf16>(p, dw, st);
  }
  return hipErrorInvalidValue;
}

template <int D, typename IO>
static hipError_t launch_act_t(const BwdActParams& p, float* dA_log, float* ddt_bias, hipStream_t st) {
  const int ng = bwd_act_groups(p.tokens, D);
  hipLaunchKernelGGL((kda_bwd_act_kernel<D, IO>), dim3((unsigned)ng, (unsigned)p.H), dim3(256), 0, st, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (p.f == nullptr) return hipSuccess;
  if (hipError_t e = launch_sum(p.ddt_part, ddt_bias, (size_t)p.H * D, ng, st); e != hipSuccess) return e;
  return launch_sum(p.dA_part, dA_log, (size_t)p.H, ng, st);
}

hipError_t launch_bwd_act(const BwdActParams& p, float* dA_log, float* ddt_bias, int D, bool fp32,
                          hipStream_t st) {
  if (p.tokens <= 0) return hipSuccess;
  switch (D) {
    case 16: return fp32 ? launch_act_t<16, float>(p, dA_log, ddt_bias, st) : launch_act_t<16, __bf16>(p, dA_log, ddt_bias, st);
    case 32: return fp32 ? launch_act_t<32, float>(p, dA_log, ddt_bias, st) : launch_act_t<32, __bf16>(p, dA_log, ddt_bias, st);
    case 64: return fp32 ? launch_act_t<64, float>(p, dA_log, ddt_bias, st) : launch_act_t<64, __bf16>(p, dA_log, ddt_bias, st);
    case 128: return fp32 ? launch_act_t<128, float>(p, dA_log, ddt_bias, st) : launch_act_t<128, __bf16>(p, dA_log, ddt_bias, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
