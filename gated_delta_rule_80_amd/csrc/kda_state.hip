// State walk of the KDA prefill: one workgroup per (sequence, head, block of VB
// value columns), walking the chunks of the sequence in order.  Value columns of
// the state evolve independently (every product below is column-wise in v), so
// splitting them across workgroups is exact and gives B*H*(D/VB) parallel walks.
//
// Per chunk, with S the D x VB float32 state block at the chunk start and the
// chunk record written by the preparation kernel:
//   U      = U~ - W S                         (the chunk's corrected new values)
//   O      = (scale Q Lambda) S + P U         (inter-chunk + intra-chunk output)
//   S_next = Diag(Lambda_C) S + Ktil^T U      (Ktil = K exp(Gamma_C - Gamma))
// S stays in float32 matrix-core accumulators for the whole walk; a copy in the
// operand element type is staged in LDS for the products that read it.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

constexpr int kStateThreads = 256;

// acc += P(rows i0..i0+15, k) * B(k, 16 cols), P read from global row-major with
// the causal mask j <= i applied in registers; only k < i0 + 16 is visited.
template <int C>
__device__ __forceinline__ void mma_causal(f32x4& acc, const __bf16* P, int i0, const __bf16* Bt,
                                           int ldb, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int i = i0 + r;
  if constexpr (C % 32 == 0) {
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) {
      if (k0 < i0 + 16) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(P + (size_t)i * C + k0 + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + 8 * g + e > i) a[e] = (__bf16)0.f;
        bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k0 + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 16) {
      if (k0 < i0 + 16) {
        bf16x4 a = *reinterpret_cast<const bf16x4*>(P + (size_t)i * C + k0 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k0 + 4 * g + e > i) a[e] = (__bf16)0.f;
        s16x4 as = __builtin_bit_cast(s16x4, a);
        s16x4 bs = *reinterpret_cast<const s16x4*>(Bt + r * ldb + k0 + 4 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as, bs, acc, 0, 0, 0);
      }
    }
  }
}
template <int C>
__device__ __forceinline__ void mma_causal(f32x4& acc, const float* P, int i0, const float* Bt,
                                           int ldb, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int i = i0 + r;
#pragma unroll
  for (int k0 = 0; k0 < C; k0 += 4) {
    if (k0 < i0 + 16) {
      const int kk = k0 + g;
      const float a = (kk <= i) ? P[(size_t)i * C + kk] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Bt[r * ldb + kk], acc, 0, 0, 0);
    }
  }
}

template <int D, int C, int VB, typename IO, typename E>
__global__ __launch_bounds__(kStateThreads) void kda_chunk_state_kernel(StateParams p) {
  constexpr int PE = 16 / (int)sizeof(E);
  constexpr int LS = D + PE;  // sS row stride: row = value column v, k = key channel c
  constexpr int LU = C + PE;  // sU row stride: row = value column v, k = token t
  constexpr int NV = D / VB;
  constexpr int VT = VB / 16;
  constexpr int T1 = (C / 16) * VT;  // U / O tiles (t-tile, v-tile)
  constexpr int T3 = (D / 16) * VT;  // state tiles (c-tile, v-tile)
  constexpr int P1 = (T1 + 3) / 4;
  constexpr int P3 = (T3 + 3) / 4;
  constexpr RecordLayout RL = record_layout(C, D, sizeof(E));
  __shared__ __attribute__((aligned(16))) E sS[VB * LS];
  __shared__ __attribute__((aligned(16))) E sU[VB * LU];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  // Workgroups of one head's value blocks are placed on the same XCD (dispatch
  // is round robin over the 8 XCDs), so they share the chunk records in L2.
  const int total = p.B * p.H * NV;
  int bh, vblk;
  if (total % (8 * NV) == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    vblk = slot % NV;
    bh = (slot / NV) * 8 + xcd;
  } else {
    vblk = blockIdx.x % NV;
    bh = blockIdx.x / NV;
  }
  const int h = bh % p.H, b = bh / p.H;
  const int vb0 = vblk * VB;

  // ---- initial state
  f32x4 accS[P3];
  const size_t sbase = (size_t)bh * D * D;
#pragma unroll
  for (int i = 0; i < P3; ++i) {
    const int tt = wave + 4 * i;
    accS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tt < T3 && p.S0 != nullptr) {
      const int Ct = tt / VT, Vt = tt % VT;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        accS[i][e] = p.S0[sbase + (size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r];
    }
  }
  auto stage_state = [&]() {
#pragma unroll
    for (int i = 0; i < P3; ++i) {
      const int tt = wave + 4 * i;
      if (tt < T3) {
        const int Ct = tt / VT, Vt = tt % VT;
        store4(&sS[(16 * Vt + r) * LS + 16 * Ct + 4 * g4], accS[i][0], accS[i][1], accS[i][2],
               accS[i][3]);
      }
    }
  };
  stage_state();

  IO* o = static_cast<IO*>(p.o);
  const size_t HD = (size_t)p.H * D;
  for (int n = 0; n < p.NT; ++n) {
    const char* recp = p.ws + ((size_t)bh * p.NT + n) * RL.bytes;
    const E* W = reinterpret_cast<const E*>(recp) + RL.w;
    const E* QL = reinterpret_cast<const E*>(recp) + RL.ql;
    const E* KT = reinterpret_cast<const E*>(recp) + RL.kt;
    const E* Ut = reinterpret_cast<const E*>(recp) + RL.u;
    const E* P = reinterpret_cast<const E*>(recp) + RL.p;
    const float* LC = reinterpret_cast<const float*>(recp + RL.lc_bytes);
    __syncthreads();  // sS holds this chunk's starting state; sU is free
    f32x4 accO[P1];
    // ---- U = U~ - W S,  O = QL S
#pragma unroll
    for (int i = 0; i < P1; ++i) {
      const int tt = wave + 4 * i;
      accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (tt < T1) {
        const int R = tt / VT, Vt = tt % VT;
        f32x4 ws = {0.f, 0.f, 0.f, 0.f};
        mma_rows<D>(ws, W + (size_t)16 * R * D, D, sS + 16 * Vt * LS, LS, lane);
        mma_rows<D>(accO[i], QL + (size_t)16 * R * D, D, sS + 16 * Vt * LS, LS, lane);
        float u[4];
        load4(Ut + ((size_t)(R * (D / 16) + vb0 / 16 + Vt) * 64 + lane) * 4, u);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] -= ws[e];
        store4(&sU[(16 * Vt + r) * LU + 16 * R + 4 * g4], u[0], u[1], u[2], u[3]);
      }
    }
    __syncthreads();  // sU complete; every read of sS for this chunk is done
    // ---- O += P U, write O
#pragma unroll
    for (int i = 0; i < P1; ++i) {
      const int tt = wave + 4 * i;
      if (tt < T1) {
        const int R = tt / VT, Vt = tt % VT;
        mma_causal<C>(accO[i], P, 16 * R, sU + 16 * Vt * LU, LU, lane);
        const int v = vb0 + 16 * Vt + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = n * C + 16 * R + 4 * g4 + e;
          if (t < p.T) o[((size_t)b * p.T + t) * HD + (size_t)h * D + v] = from_f32<IO>(accO[i][e]);
        }
      }
    }
    // ---- S = Diag(Lambda_C) S + Ktil^T U
#pragma unroll
    for (int i = 0; i < P3; ++i) {
      const int tt = wave + 4 * i;
      if (tt < T3) {
        const int Ct = tt / VT, Vt = tt % VT;
        const f32x4 lc = *reinterpret_cast<const f32x4*>(LC + 16 * Ct + 4 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] *= lc[e];
        mma_rows<C>(accS[i], KT + (size_t)16 * Ct * C, C, sU + 16 * Vt * LU, LU, lane);
      }
    }
    stage_state();
  }
  // ---- final state
  if (p.S_T != nullptr) {
#pragma unroll
    for (int i = 0; i < P3; ++i) {
      const int tt = wave + 4 * i;
      if (tt < T3) {
        const int Ct = tt / VT, Vt = tt % VT;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.S_T[sbase + (size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r] = accS[i][e];
      }
    }
  }
}

template <int D, int C, typename IO, typename E>
static hipError_t launch_state_t(const StateParams& p, int vb, hipStream_t st) {
  constexpr int VBmax = D >= 64 ? 64 : D;
  if (vb == 32 && D >= 32) {
    constexpr int VB = D >= 32 ? 32 : D;
    const unsigned grid = (unsigned)((size_t)p.B * p.H * (D / VB));
    hipLaunchKernelGGL((kda_chunk_state_kernel<D, C, VB, IO, E>), dim3(grid),
                       dim3(kStateThreads), 0, st, p);
  } else {
    const unsigned grid = (unsigned)((size_t)p.B * p.H * (D / VBmax));
    hipLaunchKernelGGL((kda_chunk_state_kernel<D, C, VBmax, IO, E>), dim3(grid),
                       dim3(kStateThreads), 0, st, p);
  }
  return hipGetLastError();
}

template <int D, typename IO, typename E>
static hipError_t launch_state_c(const StateParams& p, int C, int vb, hipStream_t st) {
  switch (C) {
    case 16: return launch_state_t<D, 16, IO, E>(p, vb, st);
    case 32: return launch_state_t<D, 32, IO, E>(p, vb, st);
    case 64:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_state_t<D, 64, IO, E>(p, vb, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO, typename E>
static hipError_t launch_state_d(const StateParams& p, int D, int C, int vb, hipStream_t st) {
  switch (D) {
    case 16: return launch_state_c<16, IO, E>(p, C, vb, st);
    case 32: return launch_state_c<32, IO, E>(p, C, vb, st);
    case 64: return launch_state_c<64, IO, E>(p, C, vb, st);
    case 128: return launch_state_c<128, IO, E>(p, C, vb, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state(const StateParams& p, int D, int C, bool fp32, int vb, hipStream_t st) {
  return fp32 ? launch_state_d<float, float>(p, D, C, vb, st)
              : launch_state_d<__bf16, __bf16>(p, D, C, vb, st);
}

}  // namespace kda
