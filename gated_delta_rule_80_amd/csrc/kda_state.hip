// State walk of the KDA prefill: one workgroup per (sequence, head, block of VB
// value columns), walking the chunks of the sequence in order.  Value columns of
// the state evolve independently (every product below is column-wise in v), so
// splitting them across workgroups is exact and gives B*H*(D/VB) parallel walks.
//
// Per chunk, with S the D x VB float32 state block at the chunk start and the
// chunk record written by the preparation kernel:
//   U      = U~ - W S                         (the chunk's corrected new values)
//   O^T    = S^T (scale Q Lambda)^T + U^T P^T (inter-chunk + intra-chunk output)
//   S_next = Diag(Lambda_C) S + Ktil^T U      (Ktil = K exp(Gamma_C - Gamma))
// S stays in float32 matrix-core accumulators for the whole walk; a copy in the
// operand element type is staged in LDS for the products that read it.  The
// output is formed transposed so each lane holds 4 consecutive value columns of
// one token, which it stores contiguously.
//
// The chunk record of chunk n+1 is loaded into registers while chunk n is being
// computed, so the serial walk does not wait on memory latency.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

constexpr int kStateThreads = 256;

template <typename E, int D, int C, int NCTW, int NU>
struct ChunkRegs {
  RowFrag<E, D> w;         // W rows of this wave's t-tile
  RowFrag<E, D> ql;        // scale Q Lambda rows of this wave's t-tile
  RowFrag<E, C> p;         // P rows of this wave's t-tile (causally masked)
  RowFrag<E, C> kt[NCTW];  // Ktil^T rows of this wave's c-tiles
  f32x4 ut[NU];            // U~ fragments of this wave's (t-tile, v-tile) units
  f32x4 lc[NCTW];          // Lambda_C for the 4 rows this lane holds per c-tile
};

template <int D, int C, int VB, typename IO, typename E>
__global__ __launch_bounds__(kStateThreads) void kda_chunk_state_kernel(StateParams p) {
  constexpr int PE = 16 / (int)sizeof(E);
  constexpr int LS = D + PE;  // sS row stride: row = value column v, k = key channel c
  constexpr int LU = C + PE;  // sU row stride: row = value column v, k = token t
  constexpr int NV = D / VB;
  constexpr int VT = VB / 16;   // v-tiles
  constexpr int RT = C / 16;    // t-tiles
  constexpr int CT = D / 16;    // c-tiles
  static_assert(4 % RT == 0 || RT == 4, "t-tiles must divide the 4 waves");
  constexpr int NU = (RT * VT + 3) / 4;      // (t-tile, v-tile) units per wave (upper bound)
  constexpr int NS = (CT * VT + 3) / 4;      // (c-tile, v-tile) units per wave (upper bound)
  constexpr int CTW = CT < 4 ? CT : 4;       // c-tile stride between a wave's units
  constexpr int NCTW = CT > 4 ? CT / 4 : 1;  // distinct c-tiles per wave
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

  // this wave's tiles
  const int R = wave % RT;               // t-tile of every (t, v) unit of this wave
  const bool has_u = wave < RT * VT;     // any (t, v) unit at all
  const int i_row = 16 * R + r;          // row of P / W / QL this lane reads
  const int csteps = (16 * R + 16 + RowFrag<E, C>::STEP - 1) / RowFrag<E, C>::STEP;

  auto load_chunk = [&](int n, ChunkRegs<E, D, C, NCTW, NU>& cr) {
    const char* recp = p.ws + ((size_t)bh * p.NT + n) * RL.bytes;
    const E* W = reinterpret_cast<const E*>(recp) + RL.w;
    const E* QL = reinterpret_cast<const E*>(recp) + RL.ql;
    const E* KT = reinterpret_cast<const E*>(recp) + RL.kt;
    const E* Ut = reinterpret_cast<const E*>(recp) + RL.u;
    const E* P = reinterpret_cast<const E*>(recp) + RL.p;
    const float* LC = reinterpret_cast<const float*>(recp + RL.lc_bytes);
    if (has_u) {
      cr.w.load(W + (size_t)i_row * D, g4);
      cr.ql.load(QL + (size_t)i_row * D, g4);
      cr.p.load(P + (size_t)i_row * C, g4);
    }
#pragma unroll
    for (int j = 0; j < NCTW; ++j) {
      const int Ct = (wave % CTW) + 4 * j;
      cr.kt[j].load(KT + (size_t)(16 * Ct + r) * C, g4);
      cr.lc[j] = *reinterpret_cast<const f32x4*>(LC + 16 * Ct + 4 * g4);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + 4 * i;
      if (u < RT * VT) {
        const int Vt = u / RT;
        float t4[4];
        load4(Ut + ((size_t)(R * (D / 16) + vb0 / 16 + Vt) * 64 + lane) * 4, t4);
        cr.ut[i] = f32x4{t4[0], t4[1], t4[2], t4[3]};
      }
    }
  };

  // ---- initial state
  f32x4 accS[NS];
  const size_t sbase = (size_t)bh * D * D;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = wave + 4 * i;
    accS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (u < CT * VT && p.S0 != nullptr) {
      const int Ct = u % CT, Vt = u / CT;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        accS[i][e] = p.S0[sbase + (size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r];
    }
  }
  auto stage_state = [&]() {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + 4 * i;
      if (u < CT * VT) {
        const int Ct = u % CT, Vt = u / CT;
        store4(&sS[(16 * Vt + r) * LS + 16 * Ct + 4 * g4], accS[i][0], accS[i][1], accS[i][2],
               accS[i][3]);
      }
    }
  };
  stage_state();

  IO* o = static_cast<IO*>(p.o);
  const size_t HD = (size_t)p.H * D;
  ChunkRegs<E, D, C, NCTW, NU> cur, nxt;
  load_chunk(0, cur);
  for (int n = 0; n < p.NT; ++n) {
    if (n + 1 < p.NT) load_chunk(n + 1, nxt);
    if (has_u) cur.p.mask_above(i_row, g4);
    __syncthreads();  // sS holds this chunk's starting state; sU is free
    // ---- U = U~ - W S  and  O^T = S^T QL^T
    f32x4 accO[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + 4 * i;
      accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < RT * VT) {
        const int Vt = u / RT;
        RowFrag<E, D> sf;
        sf.load(sS + (16 * Vt + r) * LS, g4);
        f32x4 ws = {0.f, 0.f, 0.f, 0.f};
        mma<D>(ws, cur.w, sf);        // (t, v) tile of W S
        mma<D>(accO[i], sf, cur.ql);  // (v, t) tile of S^T QL^T
        store4(&sU[(16 * Vt + r) * LU + 16 * R + 4 * g4], cur.ut[i][0] - ws[0],
               cur.ut[i][1] - ws[1], cur.ut[i][2] - ws[2], cur.ut[i][3] - ws[3]);
      }
    }
    __syncthreads();  // sU complete; every read of sS for this chunk is done
    // ---- O^T += U^T P^T (j <= i), store O
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + 4 * i;
      if (u < RT * VT) {
        const int Vt = u / RT;
        RowFrag<E, C> uf;
        uf.load(sU + (16 * Vt + r) * LU, g4);
        mma<C>(accO[i], uf, cur.p, csteps);
        const int t = n * C + 16 * R + r;
        if (t < p.T)
          store4(o + ((size_t)b * p.T + t) * HD + (size_t)h * D + vb0 + 16 * Vt + 4 * g4,
                 accO[i][0], accO[i][1], accO[i][2], accO[i][3]);
      }
    }
    // ---- S = Diag(Lambda_C) S + Ktil^T U
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + 4 * i;
      if (u < CT * VT) {
        const int Vt = u / CT;
        const int j = i % NCTW;  // this unit's c-tile is (wave % CTW) + 4 * j
        RowFrag<E, C> uf;
        uf.load(sU + (16 * Vt + r) * LU, g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] *= cur.lc[j][e];
        mma<C>(accS[i], cur.kt[j], uf);
      }
    }
    stage_state();
    cur = nxt;
  }
  // ---- final state
  if (p.S_T != nullptr) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + 4 * i;
      if (u < CT * VT) {
        const int Ct = u % CT, Vt = u / CT;
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
