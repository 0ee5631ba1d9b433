// Split state walk: the segment maps and the composition of the segment start
// states (the segment walks themselves are the state walk kernel's).
//
// Over a run of chunks the recurrence S_next = Diag(Lambda_C) S + Ktil^T (U~ - W S)
// is affine in the state it starts from, S_end = M S_start + N: N is the end
// state walked from zero, and M's columns are the end states walked from the
// identity's columns with U~ taken as zero.  A (sequence, head) whose chain of
// chunk steps is long next to the number of walks running is cut into segments;
// the N and M of every segment but the last are walked in parallel, the start
// states are composed in order (one D x D product per segment), and every
// segment is then walked with its outputs from its own start.  The composition
// is exact in exact arithmetic; only the rounding order differs from one long
// walk.  The backward's reverse walk composes the gradients of the segments'
// end states the same way with the transposed maps (its map walks live with
// the reverse walk kernel; the composition is the kernel below, reversed).
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

// The part of a chunk record a map walk reads, copied into LDS.  Byte offsets;
// every part is a whole number of 16-byte chunks.
template <int D, int C, int VB, typename E>
struct MapImage {
  static constexpr int ES = (int)sizeof(E);
  static constexpr int W = 0;                // [C][D] swizzled
  static constexpr int KT = W + C * D * ES;  // [D][C] swizzled
  static constexpr int U = KT + D * C * ES;  // (C/16) x (VB/16) fragment tiles
  static constexpr int LC = U + C * VB * ES; // [D] float
  static constexpr int BYTES = LC + D * 4;
  static constexpr int CHUNKS = BYTES / 16;
  static_assert(BYTES % 16 == 0, "record image is whole 16-byte chunks");
};

// One workgroup per (sequence, head, segment s < nseg - 1, kind, block of VB
// columns): kind 0 walks the segment's chunks from zero (from S0 when s = 0)
// with the chunk inputs and writes N; kind 1 (s >= 1) walks them from the
// identity's columns vb0 .. vb0 + VB - 1 without inputs and writes those rows of
// Mt.  The wave layout, record copy and products are the state walk's, without
// the output and its operands (Q Lambda, P).
template <int D, int C, int VB, typename E, int NT>
__global__ __launch_bounds__(NT, 2) void kda_seg_map_kernel(SplitParams p) {
  constexpr int NW = NT / 64;
  constexpr int PE = 16 / (int)sizeof(E);
  constexpr int ES = (int)sizeof(E);
  constexpr int LS = D + PE;  // sS row stride: row = column v, k = key channel c
  constexpr int LU = C + PE;  // sU row stride: row = column v, k = token t
  constexpr int NV = D / VB;
  constexpr int VT = VB / 16;
  constexpr int RT = C / 16;
  constexpr int CT = D / 16;
  static_assert(NW % RT == 0, "every unit of a wave has the same t-tile");
  static_assert(CT <= NW || CT % NW == 0, "every unit of a wave has one of NCTW c-tiles");
  constexpr int NU = (RT * VT + NW - 1) / NW;
  constexpr int NS = (CT * VT + NW - 1) / NW;
  constexpr int CTW = CT < NW ? CT : NW;
  constexpr int NCTW = CT > NW ? CT / NW : 1;
  constexpr bool FULL_U = (RT * VT) % NW == 0;
  constexpr bool FULL_S = (CT * VT) % NW == 0;
  constexpr RecordLayout RL = record_layout(C, D, sizeof(E));
  using IMG = MapImage<D, C, VB, E>;
  __shared__ __attribute__((aligned(16))) char img[IMG::BYTES];
  __shared__ __attribute__((aligned(16))) E sS[VB * LS];
  __shared__ __attribute__((aligned(16))) E sU[VB * LU];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  // (head, segment) groups of 2 NV workgroups, numbered XCD by XCD: the
  // workgroups of one group read the same records
  const int nmap = p.whole ? p.nseg : p.nseg - 1;  // segments with maps
  const int pos = xcd_major(blockIdx.x, gridDim.x);
  const int job = pos % (2 * NV), grp = pos / (2 * NV);
  const int kind = job / NV, vblk = job % NV;
  const int bh = grp / nmap, s = grp % nmap;
  if (kind == 1 && s == 0 && !p.whole) return;  // the walk's first segment needs no M
  const int vb0 = vblk * VB;
  // every segment but the last has seg_len whole chunks; the last (only mapped
  // for a whole call) has the rest, its last chunk possibly partial
  const int nch = p.whole && s == nmap - 1 ? p.nch - s * p.seg_len : p.seg_len;
  // chunk n of the segment is record rec0 + n rstride (rec_slot)
  const size_t rstride = (size_t)p.B * p.H;
  const size_t rec0 = rec_slot((size_t)s * p.seg_len, bh, rstride);

  const int R = wave % RT;
  const bool has_u = FULL_U || wave < RT * VT;
  const int i_row = 16 * R + r;

  // ---- record copy (W, Ktil^T, U~ of this block, Lambda_C), as in the state walk
  constexpr int ITERS = (IMG::CHUNKS + NT - 1) / NT;
  uint32_t src_off[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    constexpr int RCD = D * ES / 16;
    constexpr int RCC = C * ES / 16;
    constexpr int UPIECE = VT * 64 * 4 * ES / 16;
    const int idx = it * NT + tid;
    const int byte = idx * 16;
    size_t off;
    if (byte < IMG::KT) {
      const int row = idx / RCD, cs = idx % RCD;
      off = (size_t)RL.w * ES + (size_t)(row * RCD + (cs ^ (row & (RCD - 1)))) * 16;
    } else if (byte < IMG::U) {
      const int ci = idx - IMG::KT / 16;
      const int row = ci / RCC, cs = ci % RCC;
      off = (size_t)RL.kt * ES + (size_t)(row * RCC + (cs ^ (row & (RCC - 1)))) * 16;
    } else if (byte < IMG::LC) {
      const int ci = idx - IMG::U / 16;
      const int tt = ci / UPIECE, w = ci % UPIECE;
      off = (size_t)RL.u * ES + ((size_t)(tt * (D / 16) + vb0 / 16) * 64 * 4) * ES + (size_t)w * 16;
    } else {
      off = RL.lc_bytes + (size_t)(idx - IMG::LC / 16) * 16;
    }
    src_off[it] = (uint32_t)off;
  }
  const bool skip_u = kind == 1;  // no inputs: U~ is never read, so never copied
  auto issue_copy = [&](int n) {
    const char* recp = p.ws + (rec0 + n * rstride) * RL.bytes;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int idx = it * NT + tid;
      const int byte = idx * 16;
      if (idx < IMG::CHUNKS && !(skip_u && byte >= IMG::U && byte < IMG::LC))
        __builtin_amdgcn_global_load_lds((const glb_void_t*)(recp + src_off[it]),
                                         (lds_void_t*)(img + (size_t)(it * NT + 64 * wave) * 16), 16,
                                         0, 0);
    }
  };

  // ---- initial state: S0, zero or the identity's columns
  f32x4 accS[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = wave + NW * i;
    accS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (FULL_S || u < CT * VT) {
      const int Ct = u % CT, Vt = u / CT;
      const int v = vb0 + 16 * Vt + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 16 * Ct + 4 * g4 + e;
        if (kind == 1)
          accS[i][e] = c == v ? 1.f : 0.f;
        else if (s == 0 && !p.whole && p.S0 != nullptr)
          accS[i][e] = p.S0[(size_t)bh * D * D + (size_t)c * D + v];
      }
    }
  }
  auto stage_state = [&]() {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (FULL_S || u < CT * VT) {
        const int Ct = u % CT, Vt = u / CT;
        store4(&sS[(16 * Vt + r) * LS + 16 * Ct + 4 * g4], accS[i][0], accS[i][1], accS[i][2],
               accS[i][3]);
      }
    }
  };
  stage_state();

  const E* iW = reinterpret_cast<const E*>(img + IMG::W);
  const E* iKT = reinterpret_cast<const E*>(img + IMG::KT);
  const E* iU = reinterpret_cast<const E*>(img + IMG::U);
  const float* iLC = reinterpret_cast<const float*>(img + IMG::LC);

  if (nch > 0) issue_copy(0);
  for (int n = 0; n < nch; ++n) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of chunk n
    lds_barrier();                  // the whole image of chunk n and the state are in LDS
    RowFrag<E, D> fw;
    RowFrag<E, C> fkt[NCTW];
    f32x4 flc[NCTW];
    f32x4 fu[NU];
    if (has_u) load_swz<D>(fw, iW, i_row, g4);
#pragma unroll
    for (int j = 0; j < NCTW; ++j) {
      const int Ct = (wave % CTW) + CTW * j;
      load_swz<C>(fkt[j], iKT, 16 * Ct + r, g4);
      flc[j] = *reinterpret_cast<const f32x4*>(iLC + 16 * Ct + 4 * g4);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      fu[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if ((FULL_U || u < RT * VT) && kind == 0)
        fu[i] = load4v(iU + ((size_t)(R * VT + u / RT) * 64 + lane) * 4);
    }
    lds_barrier();  // every wave holds its fragments: the image may be overwritten
    if (n + 1 < nch) issue_copy(n + 1);
    // ---- U = U~ - W S
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (FULL_U || u < RT * VT) {
        const int Vt = u / RT;
        RowFrag<E, D> sf;
        sf.load(sS + (16 * Vt + r) * LS, g4);
        f32x4 ws = {0.f, 0.f, 0.f, 0.f};
        mma<D>(ws, fw, sf);
        store4(&sU[(16 * Vt + r) * LU + 16 * R + 4 * g4], fu[i][0] - ws[0], fu[i][1] - ws[1],
               fu[i][2] - ws[2], fu[i][3] - ws[3]);
      }
    }
    lds_barrier();  // sU complete; every read of sS for this chunk is done
    // ---- S = Diag(Lambda_C) S + Ktil^T U
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (FULL_S || u < CT * VT) {
        const int Vt = u / CT;
        const int j = i % NCTW;
        RowFrag<E, C> uf;
        uf.load(sU + (16 * Vt + r) * LU, g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] *= flc[j][e];
        mma<C>(accS[i], fkt[j], uf);
      }
    }
    stage_state();
  }
  // ---- N or M row-major, and the rows vb0 .. of Mt (4 consecutive key channels
  // a lane)
  float* slots = p.maps + (size_t)grp * 3 * D * D;
  float* out = slots + (kind == 1 ? 2 : 0) * (size_t)D * D;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = wave + NW * i;
    if (FULL_S || u < CT * VT) {
      const int Ct = u % CT, Vt = u / CT;
      const int c = 16 * Ct + 4 * g4, v = vb0 + 16 * Vt + r;
      if (kind == 1)
        store4(slots + (size_t)D * D + (size_t)v * D + c, accS[i][0], accS[i][1], accS[i][2],
               accS[i][3]);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(size_t)(c + e) * D + v] = accS[i][e];
    }
  }
}

// The composition kernels' layout: one workgroup per (sequence, head, block of
// CW columns); thread (row group rg, column col) holds rows rg RPT .. rg RPT +
// RPT - 1 of its column.
template <int D>
struct ComposeShape {
  static constexpr int CW = D >= 64 ? 8 : 16;  // columns per workgroup
  static constexpr int NCB = D / CW;
  static constexpr int RG = 256 / CW;          // row groups
  static constexpr int RPT = D / RG;           // rows per thread
  static_assert(RPT >= 1 && RPT * RG == D, "rows split evenly");
};

// acc += (A X)[rows c0 .., column col], A held as A[k][row] (D x D float32 in
// global memory, copied into sA whole), X the workgroup's D x CW column block in
// sX.  Every thread calls it; it ends with the barrier after the last read of sA
// and sX.
template <int D>
__device__ __forceinline__ void apply_map(const float* A, float* sA, const float* sX,
                                          float (&acc)[ComposeShape<D>::RPT], int tid, int col,
                                          int c0) {
  using SH = ComposeShape<D>;
  constexpr int CW = SH::CW, RPT = SH::RPT;
  constexpr int DD = D * D;
  const int wave = tid >> 6;
  // 16 bytes a lane; the lanes of a wave fill 64 consecutive pieces
  for (int q = 0; q < DD / 4; q += 256)
    if (q + tid < DD / 4)
      __builtin_amdgcn_global_load_lds((const glb_void_t*)(A + 4 * (size_t)(q + tid)),
                                       (lds_void_t*)(sA + 4 * (q + 64 * wave)), 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // A and X are in LDS
#pragma unroll 4
  for (int j = 0; j < D; ++j) {
    const float xj = sX[j * CW + col];
    const float* arow = sA + j * D + c0;
    if constexpr (RPT % 4 == 0) {
#pragma unroll
      for (int q = 0; q < RPT / 4; ++q) {
        const f32x4 m = *reinterpret_cast<const f32x4*>(arow + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q + e] = fmaf(m[e], xj, acc[4 * q + e]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) acc[i] = fmaf(arow[i], xj, acc[i]);
    }
  }
  __syncthreads();  // every read of sA and sX for this step is done
}

// Segment start states in order, in float32.  Forward: starts[0] = S0 (or
// zeros), starts[1] = N_0, starts[s + 1] = M_s starts[s] + N_s.  Reverse (the
// gradients of the segments' end states): starts[nseg - 1] = dS_T (or zeros),
// starts[nseg - 2] = N'_{nseg-1}, starts[s - 1] = M_s^T starts[s] + N'_s.  Both
// are X_next = A X + N with A held as A[k][row]: Mt_s for M_s, M_s row-major for
// M_s^T.
template <int D>
__global__ __launch_bounds__(256) void kda_seg_combine_kernel(SplitParams p) {
  using SH = ComposeShape<D>;
  constexpr int CW = SH::CW, NCB = SH::NCB, RPT = SH::RPT;
  __shared__ __attribute__((aligned(16))) float sA[D * D];
  __shared__ float sX[D * CW];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / NCB, cb = blockIdx.x % NCB;
  const int col = tid % CW, rg = tid / CW;
  const int v = cb * CW + col, c0 = rg * RPT;
  const int nseg = p.nseg;
  const bool rev = p.reverse != 0;
  const size_t DD = (size_t)D * D;
  float* st = p.starts + (size_t)bh * nseg * DD;
  const float* mp = p.maps + (size_t)bh * (nseg - 1) * 3 * DD;
  auto slot = [&](int s, int k) { return mp + ((size_t)s * 3 + k) * DD; };
  const int first = rev ? nseg - 1 : 0, second = rev ? nseg - 2 : 1;
  const float* n1 = slot(rev ? nseg - 2 : 0, 0);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const size_t e = (size_t)(c0 + i) * D + v;
    st[first * DD + e] = p.S0 != nullptr ? p.S0[(size_t)bh * DD + e] : 0.f;
    const float x = n1[e];
    st[second * DD + e] = x;
    sX[(c0 + i) * CW + col] = x;
  }
  for (int k = 1; k < nseg - 1; ++k) {
    const int s = rev ? nseg - 1 - k : k;
    const float* N = rev ? slot(s - 1, 0) : slot(s, 0);
    float* out = st + (size_t)(rev ? s - 1 : s + 1) * DD;
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = N[(size_t)(c0 + i) * D + v];
    apply_map<D>(slot(s, rev ? 2 : 1), sA, sX, acc, tid, col, c0);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      sX[(c0 + i) * CW + col] = acc[i];
      out[(size_t)(c0 + i) * D + v] = acc[i];
    }
  }
}

// The state map of a whole call per (sequence, head), from the maps of its
// segments in order: M = M_{P-1} ... M_1 M_0 and N = M_{P-1}(... (M_1 N_0 +
// N_1) ...) + N_{P-1}, in float32.  The columns of [M | N] evolve independently
// (X <- M_s X, plus N_s in the N columns), so workgroup (sequence, head, part,
// column block) carries one CW-column block of M (part 0) or N (part 1).
template <int D>
__global__ __launch_bounds__(256) void kda_seg_compose_kernel(SplitParams p) {
  using SH = ComposeShape<D>;
  constexpr int CW = SH::CW, NCB = SH::NCB, RPT = SH::RPT;
  __shared__ __attribute__((aligned(16))) float sA[D * D];
  __shared__ float sX[D * CW];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / (2 * NCB), part = blockIdx.x / NCB % 2, cb = blockIdx.x % NCB;
  const int col = tid % CW, rg = tid / CW;
  const int v = cb * CW + col, c0 = rg * RPT;
  const int nseg = p.nseg;
  const size_t DD = (size_t)D * D;
  const float* mp = p.maps + (size_t)bh * nseg * 3 * DD;
  auto slot = [&](int s, int k) { return mp + ((size_t)s * 3 + k) * DD; };
  const float* x0 = slot(0, part == 1 ? 0 : 2);  // N_0, or M_0 row-major
  float acc[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    acc[i] = x0[(size_t)(c0 + i) * D + v];
    sX[(c0 + i) * CW + col] = acc[i];
  }
  for (int s = 1; s < nseg; ++s) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = part == 1 ? slot(s, 0)[(size_t)(c0 + i) * D + v] : 0.f;
    apply_map<D>(slot(s, 1), sA, sX, acc, tid, col, c0);
#pragma unroll
    for (int i = 0; i < RPT; ++i) sX[(c0 + i) * CW + col] = acc[i];
  }
  float* out = (part == 1 ? p.N_out : p.M_out) + (size_t)bh * DD;
#pragma unroll
  for (int i = 0; i < RPT; ++i) out[(size_t)(c0 + i) * D + v] = acc[i];
}

// The state map of an empty call: M = I, N = 0, for n_mats (sequence, head) pairs.
__global__ __launch_bounds__(256) void kda_state_map_identity_kernel(float* M, float* N, size_t n, int D) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t e = i % ((size_t)D * D);
    M[i] = e / D == e % D ? 1.f : 0.f;
    N[i] = 0.f;
  }
}

template <int D, int C, typename E>
static hipError_t launch_maps_t(const SplitParams& p, int vb, int threads, hipStream_t st) {
  const size_t groups = (size_t)p.B * p.H * (p.whole ? p.nseg : p.nseg - 1);
  if (p.reverse != 0) return hipErrorInvalidValue;
  if constexpr (D == 128) {
    if (vb == 64 && threads == 512) {
      hipLaunchKernelGGL((kda_seg_map_kernel<D, C, 64, E, 512>), dim3((unsigned)(groups * 2 * 2)),
                         dim3(512), 0, st, p);
      return hipGetLastError();
    }
  }
  if (threads != 256) return hipErrorInvalidValue;
  constexpr int VBmax = D >= 64 ? 64 : D;
  if (vb == 32 && D >= 32) {
    constexpr int VB = D >= 32 ? 32 : D;
    hipLaunchKernelGGL((kda_seg_map_kernel<D, C, VB, E, 256>), dim3((unsigned)(groups * 2 * (D / VB))),
                       dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((kda_seg_map_kernel<D, C, VBmax, E, 256>),
                       dim3((unsigned)(groups * 2 * (D / VBmax))), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

template <int D, typename E>
static hipError_t launch_maps_c(const SplitParams& p, int C, int vb, int threads, hipStream_t st) {
  switch (C) {
    case 16: return launch_maps_t<D, 16, E>(p, vb, threads, st);
    case 32: return launch_maps_t<D, 32, E>(p, vb, threads, st);
    case 64:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_maps_t<D, 64, E>(p, vb, threads, st);
  }
  return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_maps_d(const SplitParams& p, int D, int C, int vb, int threads, hipStream_t st) {
  switch (D) {
    case 16: return launch_maps_c<16, E>(p, C, vb, threads, st);
    case 32: return launch_maps_c<32, E>(p, C, vb, threads, st);
    case 64: return launch_maps_c<64, E>(p, C, vb, threads, st);
    case 128: return launch_maps_c<128, E>(p, C, vb, threads, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_split_maps(const SplitParams& p, int D, int C, bool fp32, int vb, int threads,
                             hipStream_t st) {
  if (p.nseg < (p.whole ? 1 : 2)) return hipErrorInvalidValue;
  return fp32 ? launch_maps_d<float>(p, D, C, vb, threads, st)
              : launch_maps_d<__bf16>(p, D, C, vb, threads, st);
}

hipError_t launch_split_combine(const SplitParams& p, int D, hipStream_t st) {
  if (p.nseg < 2) return hipErrorInvalidValue;
  const size_t bh = (size_t)p.B * p.H;
  switch (D) {
    case 16: hipLaunchKernelGGL((kda_seg_combine_kernel<16>), dim3((unsigned)(bh * ComposeShape<16>::NCB)), dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL((kda_seg_combine_kernel<32>), dim3((unsigned)(bh * ComposeShape<32>::NCB)), dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((kda_seg_combine_kernel<64>), dim3((unsigned)(bh * ComposeShape<64>::NCB)), dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((kda_seg_combine_kernel<128>), dim3((unsigned)(bh * ComposeShape<128>::NCB)), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_state_map(const SplitParams& p, int D, int C, bool fp32, int vb, int threads,
                            hipStream_t st) {
  if (!p.whole || p.nseg < 1) return hipErrorInvalidValue;
  if (hipError_t e = launch_split_maps(p, D, C, fp32, vb, threads, st); e != hipSuccess) return e;
  const unsigned grid = (unsigned)((size_t)p.B * p.H * 2);
  switch (D) {
    case 16: hipLaunchKernelGGL((kda_seg_compose_kernel<16>), dim3(grid * ComposeShape<16>::NCB), dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL((kda_seg_compose_kernel<32>), dim3(grid * ComposeShape<32>::NCB), dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((kda_seg_compose_kernel<64>), dim3(grid * ComposeShape<64>::NCB), dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((kda_seg_compose_kernel<128>), dim3(grid * ComposeShape<128>::NCB), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_state_map_identity(float* M, float* N, size_t n, int D, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(kda_state_map_identity_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, st, M, N, n, D);
  return hipGetLastError();
}

}  // namespace kda
