// One decode step of the KDA mixer for B sequences: one workgroup per
// (sequence, head).  The D x D float32 state is streamed from HBM once, updated
// in registers and streamed back once; everything else is small.
//
//   conv ring: y = SiLU(w3 x_t + w2 x_{t-1} + w1 x_{t-2} + w0 x_{t-3}), state <- (x_{t-2}, x_{t-1}, x_t)
//   q, k L2-normalised (q also scaled);  alpha = exp(g)
//   S_bar = Diag(alpha) S;  r_k = S_bar^T k;  r_q = S_bar^T q   (one sweep over S)
//   u = beta (v - r_k);  o = r_q + (k . q) u  ( = S_new^T q );  S_new = S_bar + k u^T
// The two reductions over the key channels share one pass: each thread owns a
// few state rows x 4 value columns and partial sums are combined through LDS.
// Optional stages: g and beta from raw projections (-exp(A_log) softplus(f +
// dt_bias), sigmoid(b)), and o <- RMSNorm(o) * gain * sigmoid(gate) over the
// head's D values, which this workgroup holds whole.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

template <int D>
struct DecodeShape {
  static constexpr int NTH = (D * D / 4 < 256) ? D * D / 4 : 256;  // threads
  static constexpr int VG = D / 4;                                  // float4 column groups
  static constexpr int CG = NTH / VG;                               // row groups
  static constexpr int R = D / CG;                                  // rows per thread
  static constexpr int NW = (NTH + 63) / 64;                        // waves
};

template <int D, typename IO>
__global__ __launch_bounds__(DecodeShape<D>::NTH) void kda_decode_kernel(DecodeParams p) {
  using SH = DecodeShape<D>;
  constexpr int VG = SH::VG, CG = SH::CG, R = SH::R, NW = SH::NW;
  static_assert(R >= 1 && CG * R == D, "decode tiling");
  __shared__ float sq[D], sk[D], sv[D], sa[D], su[D];
  __shared__ float red[3][NW];
  __shared__ float ored[NW];
  __shared__ f32x4 part[2][CG][VG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const int h = bh % p.H, b = bh / p.H;
  const int vg = tid % VG, cg = tid / VG;
  float* S = p.S + (size_t)bh * D * D;

  // issue the state loads first; they do not depend on anything below
  f32x4 st[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(cg * R + i) * D) + vg);

  // ---- front end: conv ring + SiLU, decay, beta
  const size_t HD = (size_t)p.H * D;
  float yq = 0.f, yk = 0.f, yv = 0.f;
  if (tid < D) {
    const int c = tid;
    const size_t xo = (size_t)bh * D + c;
    const IO* in[3] = {static_cast<const IO*>(p.q), static_cast<const IO*>(p.k),
                       static_cast<const IO*>(p.v)};
    float y[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const float x = to_f32(in[i][xo]);
      if (p.conv_w != nullptr) {
        IO* cs = static_cast<IO*>(p.conv_state);
        const size_t so = (((size_t)b * 3 + i) * 3) * HD + (size_t)h * D + c;
        const IO r0 = cs[so], r1 = cs[so + HD], r2 = cs[so + 2 * HD];
        const f32x4 w =
            *reinterpret_cast<const f32x4*>(p.conv_w + ((size_t)i * HD + (size_t)h * D + c) * 4);
        float acc = w[0] * to_f32(r0);
        acc = fmaf(w[1], to_f32(r1), acc);
        acc = fmaf(w[2], to_f32(r2), acc);
        acc = fmaf(w[3], x, acc);
        y[i] = silu(acc);
        // ring shift: drop the oldest raw input, append this token's
        cs[so] = r1;
        cs[so + HD] = r2;
        cs[so + 2 * HD] = in[i][xo];
      } else {
        y[i] = x;
      }
    }
    yq = y[0];
    yk = y[1];
    yv = y[2];
    float gc = to_f32(static_cast<const IO*>(p.g)[xo]);
    if (p.A_log != nullptr) gc = gate_decay(gc, p.dt_bias[(size_t)h * D + c], -__expf(p.A_log[h]));
    sa[c] = __expf(gc);
  }
  // ---- L2 norms and <q, k> over the head's D channels
  float s_qq = group_sum<64>(yq * yq), s_kk = group_sum<64>(yk * yk), s_qk = group_sum<64>(yq * yk);
  if (lane == 0) {
    red[0][wave] = s_qq;
    red[1][wave] = s_kk;
    red[2][wave] = s_qk;
  }
  __syncthreads();
  s_qq = s_kk = s_qk = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    s_qq += red[0][w];
    s_kk += red[1][w];
    s_qk += red[2][w];
  }
  const float rq = (p.l2 ? 1.0f / sqrtf(s_qq + p.eps) : 1.0f) * p.scale;
  const float rk = p.l2 ? 1.0f / sqrtf(s_kk + p.eps) : 1.0f;
  const float kq = s_qk * rq * rk;  // <k_hat, q_hat>
  if (tid < D) {
    sq[tid] = yq * rq;
    sk[tid] = yk * rk;
    sv[tid] = yv;
  }
  float beta = to_f32(static_cast<const IO*>(p.beta)[bh]);
  if (p.beta_logits) beta = sigmoid(beta);
  __syncthreads();

  // ---- one sweep: decay the rows, partial S_bar^T k and S_bar^T q
  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int c = cg * R + i;
    const float a = sa[c], kc = sk[c], qc = sq[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      st[i][e] *= a;
      pk[e] = fmaf(st[i][e], kc, pk[e]);
      pq[e] = fmaf(st[i][e], qc, pq[e]);
    }
  }
  part[0][cg][vg] = pk;
  part[1][cg][vg] = pq;
  __syncthreads();
  float ov = 0.f;
  if (tid < D) {
    const int v = tid;
    float rk_v = 0.f, rq_v = 0.f;
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      rk_v += part[0][j][v / 4][v % 4];
      rq_v += part[1][j][v / 4][v % 4];
    }
    const float u = beta * (sv[v] - rk_v);
    su[v] = u;
    ov = rq_v + kq * u;
  }
  if (p.o_norm_w != nullptr) {
    // mean square of the head's D outputs (threads >= D contribute zeros)
    const float ss = group_sum<64>(ov * ov);
    if (lane == 0) ored[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += ored[w];
    if (tid < D) ov *= p.o_norm_w[tid] / sqrtf(tot * (1.0f / D) + p.o_norm_eps);
  }
  if (tid < D) {
    if (p.o_gate != nullptr) ov *= sigmoid(to_f32(static_cast<const IO*>(p.o_gate)[(size_t)bh * D + tid]));
    static_cast<IO*>(p.o)[(size_t)bh * D + tid] = from_f32<IO>(ov);
  }
  __syncthreads();
  // ---- S_new = S_bar + k u^T, streamed back
  const f32x4 u4 = *reinterpret_cast<const f32x4*>(&su[4 * vg]);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float kc = sk[cg * R + i];
#pragma unroll
    for (int e = 0; e < 4; ++e) st[i][e] = fmaf(kc, u4[e], st[i][e]);
    __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4*>(S + (size_t)(cg * R + i) * D) + vg);
  }
}

template <int D, typename IO>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)p.B * p.H);
  hipLaunchKernelGGL((kda_decode_kernel<D, IO>), dim3(grid), dim3(DecodeShape<D>::NTH), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int D, bool fp32, hipStream_t st) {
  if (fp32) {
    switch (D) {
      case 16: return launch_decode_t<16, float>(p, st);
      case 32: return launch_decode_t<32, float>(p, st);
      case 64: return launch_decode_t<64, float>(p, st);
      case 128: return launch_decode_t<128, float>(p, st);
    }
  } else {
    switch (D) {
      case 16: return launch_decode_t<16, __bf16>(p, st);
      case 32: return launch_decode_t<32, __bf16>(p, st);
      case 64: return launch_decode_t<64, __bf16>(p, st);
      case 128: return launch_decode_t<128, __bf16>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
