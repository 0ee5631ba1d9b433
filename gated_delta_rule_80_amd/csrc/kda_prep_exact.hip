// Exact chunk preparation for the KDA prefill, used for the chunks whose decays
// are too strong for the fast preparation's factoring (it lists them in the
// workspace).  One workgroup processes listed chunks in turn.  Everything here is
// independent across chunks; the serial dependence on the state is left to the
// state walk.
//
// Per chunk (Gamma = chunk-local cumulative sum of the log-decay g, per channel;
// Lambda = exp(Gamma); all decays act on the key channels):
//   1. short conv + SiLU + L2 norm of q, k (and conv + SiLU of v)
//   2. Gamma, Lambda, the chunk decay Lambda_C
//   3. A_ij = beta_i sum_c k_ic k_jc exp(Gamma_ic - Gamma_jc)   (j < i)
//      P_ij = scale * sum_c q_ic k_jc exp(Gamma_ic - Gamma_jc)  (j <= i)
//   4. T = (I + A)^-1 (unit lower triangular)
//   5. W = T diag(beta) (K * Lambda),  U~ = T diag(beta) V
// The triangular structure is the WY/UT form of a product of generalised
// Householder factors (I - beta k k^T), which is what the delta rule composes.
//
// Step 3 without overflow: exp(Gamma_i - Gamma_j) with j < i is <= 1, but the
// split exp(Gamma_i) * exp(-Gamma_j) needed to make it a matrix product overflows
// fp32 for strong decays.  The pairs (i, j) are therefore grouped by the level of
// a binary hierarchy over the chunk at which i and j first fall into different
// halves.  At level l (segments of 2^(l+1) tokens) a pair splits as
// "j in the upper half, i in the lower half" and is factored about the last
// token r of the upper half:  exp(Gamma_i - Gamma_r) * exp(Gamma_r - Gamma_j),
// both factors <= 1.  Levels >= 4 give whole 16x16 tiles; levels 0..3 live inside
// the diagonal tiles and are masked per element.  Every pair j < i is covered by
// exactly one level.
#include "kda_convnorm.h"
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

constexpr int kPrepThreads = 256;

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Level at which 16-row blocks R > Q of a chunk separate (>= 4).
__device__ __forceinline__ int tile_level(int R, int Q) { return 4 + 31 - __clz(R ^ Q); }

template <int D, int C, typename E>
struct PrepSmem {
  static constexpr int PE = 16 / (int)sizeof(E);  // 16-byte row padding, in elements
  static constexpr int LQ = D + PE;               // rows of q, k, X, Y
  static constexpr int LG = D + 4;                // rows of Gamma (floats)
  static constexpr int LT = C + PE;               // rows of (beta K Lambda)^T, (beta V)^T, T
  static constexpr int LA = C + 4;                // rows of A and T (floats)
  static constexpr int NB = C / 16;

  E q[C * LQ];       // normalised, scaled q (later: T in E precision)
  E k[C * LQ];       // normalised k
  float gam[C * LG]; // Gamma
  E klt[D * LT];     // (diag(beta) K Lambda)^T
  E vt[D * LT];      // (diag(beta) V)^T
  // region reused by phase: segment totals -> level operands X, Y -> A, T, scratch
  static constexpr int R1_LEVELS = 2 * C * LQ * (int)sizeof(E);
  // T in E precision lives in q's space when it fits (C <= D), else after the solve scratch
  static constexpr bool TB_IN_Q = C <= D;
  static constexpr int TB_OFF = (2 * C * LA + 4 * 16 * 17) * 4;
  static constexpr int R1_SOLVE = TB_OFF + (TB_IN_Q ? 0 : C * LT * (int)sizeof(E));
  static constexpr int R1_TOT = (C / 4) * D * 4;
  static constexpr int R1 = R1_LEVELS > R1_SOLVE ? (R1_LEVELS > R1_TOT ? R1_LEVELS : R1_TOT)
                                                 : (R1_SOLVE > R1_TOT ? R1_SOLVE : R1_TOT);
  alignas(16) char r1[R1];
  float beta[C];
  float pd[C];  // diagonal of P
  alignas(16) float filt[3 * 4 * D];  // the head's conv filters [q, k, v][tap][D]
};

template <int D, int C, typename IO, typename E>
__global__ __launch_bounds__(kPrepThreads) void kda_chunk_prep_exact_kernel(PrepParams p) {
  using SM = PrepSmem<D, C, E>;
  __shared__ SM sm;
  constexpr int LQ = SM::LQ, LG = SM::LG, LT = SM::LT, LA = SM::LA, NB = SM::NB;
  constexpr int NOCT = D / 8;         // 8-channel groups per token row
  constexpr int NSEG = C / 4;         // 4-token segments
  constexpr int ITEMS = NSEG * NOCT;  // <= 256
  static_assert(ITEMS <= kPrepThreads, "tile does not fit one pass");
  constexpr RecordLayout RL = record_layout(C, D, sizeof(E));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const unsigned nlist = *p.fb_count;
  for (unsigned li = blockIdx.x; li < nlist; li += gridDim.x) {
  __syncthreads();  // the previous chunk's phase 5 is done with LDS
  const int rec = (int)p.fb_list[li];
  // b: the sequence (conv state); tok0: its first token row; Tq: its length
  int n, h, b, Tq;
  long tok0;
  if (p.seqs.bounds == nullptr) {
    // rec_slot(n, b H + h, B H)
    const int BH = p.B * p.H;
    n = rec / BH;
    const int bh = rec % BH;
    h = bh % p.H;
    b = bh / p.H;
    tok0 = (long)b * p.T;
    Tq = p.T;
  } else {
    // packed sequences: rec_slot(slot, h, H)
    const int gc = rec / p.H;
    h = rec % p.H;
    b = seq_of_slot(p.seqs.cstart, p.seqs.n_seqs, gc);
    n = gc - p.seqs.cstart[b];
    tok0 = p.seqs.bounds[b];
    Tq = p.seqs.bounds[b + 1] - p.seqs.bounds[b];
    if (n < 0 || (long)n * C >= Tq) continue;  // inconsistent tables: touch nothing
  }
  const int t0 = (p.c0 + n) * C;  // first token of the chunk in its sequence
  char* recp = p.ws + (size_t)rec * RL.bytes;
  E* gW = reinterpret_cast<E*>(recp) + RL.w;
  E* gQL = reinterpret_cast<E*>(recp) + RL.ql;
  E* gKT = reinterpret_cast<E*>(recp) + RL.kt;
  E* gU = reinterpret_cast<E*>(recp) + RL.u;
  E* gP = reinterpret_cast<E*>(recp) + RL.p;
  float* gLC = reinterpret_cast<float*>(recp + RL.lc_bytes);

  // the sequence's rows: token t of it is row tok0 + t
  const long HDl = (long)p.H * D;
  const IO* q = static_cast<const IO*>(p.q) + tok0 * HDl;
  const IO* k = static_cast<const IO*>(p.k) + tok0 * HDl;
  const IO* v = static_cast<const IO*>(p.v) + tok0 * HDl;
  const IO* gg = static_cast<const IO*>(p.g) + tok0 * HDl;
  const IO* bb = static_cast<const IO*>(p.beta) + tok0 * p.H;
  const IO* cs = p.conv_state_in == nullptr
                     ? nullptr
                     : static_cast<const IO*>(p.conv_state_in) + (long)b * 9 * HDl;

  // ---------------------------------------------------------------- phase 1
  const bool active = tid < ITEMS;
  const int s = active ? tid / NOCT : 0;
  const int j = tid % NOCT;
  const int ch = 8 * j;
  const int tf = t0 + 4 * s;  // first token of this thread's segment
  // every global load of this phase is issued before the first wait
  const bool conv = p.conv_w != nullptr;
  FilterRegs<D, kPrepThreads> fr;
  if (conv) load_filters<D, kPrepThreads>(p.conv_w, p.H, h, tid, fr);
  Raw8<IO> win[3][7];
  front_load<4, IO>(q, k, v, cs, conv, 0, Tq, p.H, D, h, ch, t0, C, tf, win);
  float gl[4][8], bt[4];
  const size_t HD = (size_t)p.H * D;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = tf + m;
    const int tc = t < Tq ? t : Tq - 1;
    load8(gg + (size_t)tc * HD + (size_t)h * D + ch, gl[m]);
    bt[m] = to_f32(bb[(size_t)tc * p.H + h]);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (conv) store_filters<D, kPrepThreads>(fr, sm.filt, tid);
  __syncthreads();  // filters are in LDS
  float yq[4][8], yk[4][8], yv[4][8], qk[4];
  front_compute<4, D, IO>(win, sm.filt, conv, ch, tf, Tq, active, p.l2 != 0, p.eps, p.scale, yq,
                          yk, yv, qk);
  // raw projections -> decay and write strength (float32); zero past the end
  const bool gact = p.A_log != nullptr;
  float gbias[8], gneg = 0.f;
  if (gact) {
    load8(p.dt_bias + (size_t)h * D + ch, gbias);
    gneg = -__expf(p.A_log[h]);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bool ok = active && tf + m < Tq;
    bt[m] = ok ? (p.beta_logits ? sigmoid(bt[m]) : bt[m]) : 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      gl[m][c] = ok ? (gact ? gate_decay(gl[m][c], gbias[c], gneg) : gl[m][c]) : 0.f;
  }
  // cumulative log-decay: within the segment, then across segments
#pragma unroll
  for (int m = 1; m < 4; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) gl[m][c] += gl[m - 1][c];
  float* tot = reinterpret_cast<float*>(sm.r1);  // [NSEG][D]
  if (active) store8(tot + s * D + ch, gl[3]);
  __syncthreads();
  float pre[8], gC[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) pre[c] = gC[c] = 0.f;
  if (active) {
    for (int s2 = 0; s2 < NSEG; ++s2) {
      float t8[8];
      load8(tot + s2 * D + ch, t8);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (s2 < s) pre[c] += t8[c];
        gC[c] += t8[c];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) gl[m][c] += pre[c];
  if (active) {
    float lamC[8], ktl[4][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) lamC[c] = __expf(gC[c]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tl = 4 * s + m;
      float lam[8], ql[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        lam[c] = __expf(gl[m][c]);
        ql[c] = yq[m][c] * lam[c];
        ktl[m][c] = yk[m][c] * __expf(gC[c] - gl[m][c]);
      }
      store8(&sm.q[tl * LQ + ch], yq[m]);
      store8(&sm.k[tl * LQ + ch], yk[m]);
      store8(&sm.gam[tl * LG + ch], gl[m]);
      store8(gQL + (size_t)tl * D + ch, ql);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sm.klt[(ch + c) * LT + tl] = from_f32<E>(bt[m] * yk[m][c] * lam[c]);
        sm.vt[(ch + c) * LT + tl] = from_f32<E>(bt[m] * yv[m][c]);
      }
      if (j == 0) {
        sm.beta[tl] = bt[m];
        sm.pd[tl] = qk[m];
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      store4(gKT + (size_t)(ch + c) * C + 4 * s, ktl[0][c], ktl[1][c], ktl[2][c], ktl[3][c]);
    if (s == 0) {
      *reinterpret_cast<f32x4*>(gLC + ch) = f32x4{lamC[0], lamC[1], lamC[2], lamC[3]};
      *reinterpret_cast<f32x4*>(gLC + ch + 4) = f32x4{lamC[4], lamC[5], lamC[6], lamC[7]};
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- phase 2
  // Tiles of A^T / P^T owned by this wave: all (R, Q) with R >= Q, round robin.
  constexpr int NTILE = NB * (NB + 1) / 2;
  constexpr int TPW = (NTILE + 3) / 4;
  f32x4 accA[TPW], accP[TPW];
  int tR[TPW], tQ[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    accA[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    accP[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int idx = wave + 4 * i, R = 0;
    while (idx > R) { idx -= R + 1; ++R; }  // idx-th lower tile in row-major order
    tR[i] = (wave + 4 * i < NTILE) ? R : -1;
    tQ[i] = idx;
  }
  E* X = reinterpret_cast<E*>(sm.r1);  // [C][LQ] row-role beta*k*f or col-role k*f
  E* Y = X + C * LQ;                   // [C][LQ] row-role q*f
  constexpr int LOGC = ilog2(C);
  for (int lev = LOGC - 1; lev >= 0; --lev) {
    const int L = 1 << lev;
    for (int it = tid; it < C * NOCT; it += kPrepThreads) {
      const int t = it / NOCT, c0 = 8 * (it % NOCT);
      const bool lower = (t >> lev) & 1;
      const int ref = lower ? ((t & ~(L - 1)) - 1) : (t | (L - 1));
      float gt[8], gr[8], kk[8], f[8];
      load8(&sm.gam[t * LG + c0], gt);
      load8(&sm.gam[ref * LG + c0], gr);
      load8(&sm.k[t * LQ + c0], kk);
      if (lower) {
        float qq[8], xr[8];
        load8(&sm.q[t * LQ + c0], qq);
        const float bta = sm.beta[t];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          f[c] = __expf(gt[c] - gr[c]);
          xr[c] = bta * kk[c] * f[c];
          qq[c] *= f[c];
        }
        store8(X + t * LQ + c0, xr);
        store8(Y + t * LQ + c0, qq);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) kk[c] *= __expf(gr[c] - gt[c]);
        store8(X + t * LQ + c0, kk);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int R = tR[i], Q = tQ[i];
      if (R < 0) continue;
      if (R != Q) {
        if (tile_level(R, Q) != lev) continue;
        // transposed tiles: rows j (upper half, column role), columns i (row role)
        mma_rows<D>(accA[i], X + 16 * Q * LQ, LQ, X + 16 * R * LQ, LQ, lane);
        mma_rows<D>(accP[i], X + 16 * Q * LQ, LQ, Y + 16 * R * LQ, LQ, lane);
      } else if (lev < 4) {
        f32x4 ta = {0.f, 0.f, 0.f, 0.f}, tp = {0.f, 0.f, 0.f, 0.f};
        mma_rows<D>(ta, X + 16 * R * LQ, LQ, X + 16 * R * LQ, LQ, lane);
        mma_rows<D>(tp, X + 16 * R * LQ, LQ, Y + 16 * R * LQ, LQ, lane);
        const int ii = 16 * R + r;  // column = i
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 16 * R + 4 * g4 + e;  // row = j
          const bool ok = ((ii >> (lev + 1)) == (jj >> (lev + 1))) && ((ii >> lev) & 1) &&
                          !((jj >> lev) & 1);
          accA[i][e] += ok ? ta[e] : 0.f;
          accP[i][e] += ok ? tp[e] : 0.f;
        }
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- phase 3
  float* sA = reinterpret_cast<float*>(sm.r1);  // [C][LA]
  float* sT = sA + C * LA;                      // [C][LA]
  float* scr = sT + C * LA;                     // [4 waves][16][17]
  for (int it = tid; it < C * LA; it += kPrepThreads) sT[it] = 0.f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int R = tR[i], Q = tQ[i];
    if (R < 0) continue;
    const int ii = 16 * R + r;
    const int jj = 16 * Q + 4 * g4;
    *reinterpret_cast<f32x4*>(&sA[ii * LA + jj]) = accA[i];
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = (jj + e == ii) ? sm.pd[ii] : accP[i][e];
    store4(gP + (size_t)ii * C + jj, pv[0], pv[1], pv[2], pv[3]);
  }
  __syncthreads();

  // ---------------------------------------------------------------- phase 4
  // diagonal 16x16 blocks by forward substitution, one column per thread
  if (tid < C) {
    const int pb = tid >> 4, col = tid & 15;
    const float* Ab = sA + (16 * pb) * LA + 16 * pb;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < i; ++jj) acc = fmaf(-Ab[i * LA + jj], x[jj], acc);
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(16 * pb + i) * LA + 16 * pb + col] = x[i];
  }
  __syncthreads();
  // off-diagonal blocks, block row by block row:
  //   T_pq = -T_pp * sum_{r=q}^{p-1} A_pr T_rq
  for (int pb = 1; pb < NB; ++pb) {
    const int qb = wave;
    float* xs = scr + wave * 16 * 17;
    if (qb < pb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int rb = qb; rb < pb; ++rb) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float a = sA[(16 * pb + r) * LA + 16 * rb + k0 + g4];
          const float bv = sT[(16 * rb + k0 + g4) * LA + 16 * qb + r];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[(4 * g4 + e) * 17 + r] = acc[e];
    }
    __syncthreads();
    if (qb < pb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const float a = sT[(16 * pb + r) * LA + 16 * pb + k0 + g4];
        const float bv = xs[(k0 + g4) * 17 + r];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * pb + 4 * g4 + e) * LA + 16 * qb + r] = -acc[e];
    }
    __syncthreads();
  }
  if (p.t_out != nullptr) {
    // backward mode: T^T in the element type
    E* to = static_cast<E*>(p.t_out) + (size_t)rec * C * C;
    for (int it = tid; it < C * C; it += kPrepThreads) {
      const int jj = it / C, i = it % C;  // to[jj][i] = T[i][jj]
      to[it] = from_f32<E>(jj <= i ? sT[i * LA + jj] : 0.f);
    }
  }
  // T in the matrix-core element type
  const E* Tb;
  int LTB;
  if constexpr (sizeof(E) == 4) {
    Tb = reinterpret_cast<const E*>(sT);
    LTB = LA;
  } else {
    E* tb = SM::TB_IN_Q ? sm.q : reinterpret_cast<E*>(sm.r1 + SM::TB_OFF);  // q no longer needed
    for (int it = tid; it < C * C; it += kPrepThreads) {
      const int i = it / C, jj = it % C;
      tb[i * LT + jj] = from_f32<E>(sT[i * LA + jj]);
    }
    Tb = tb;
    LTB = LT;
    __syncthreads();
  }

  // ---------------------------------------------------------------- phase 5
  // W^T tiles (c, i): A = (beta K Lambda)^T rows c, B^T = T rows i (j <= i)
  constexpr int NWT = (D / 16) * NB;
  for (int tt = wave; tt < NWT; tt += 4) {
    const int Ct = tt / NB, It = tt % NB;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mma_rows_upto<C>(acc, sm.klt + 16 * Ct * LT, LT, Tb + 16 * It * LTB, LTB, lane, 16 * It + 16);
    const int i = 16 * It + r, c = 16 * Ct + 4 * g4;
    store4(gW + (size_t)i * D + c, acc[0], acc[1], acc[2], acc[3]);
  }
  // U~ tiles (i, v): A = T rows i, B^T = (beta V)^T rows v; stored in fragment order
  for (int tt = wave; tt < NWT; tt += 4) {
    const int It = tt / (D / 16), Vt = tt % (D / 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mma_rows_upto<C>(acc, Tb + 16 * It * LTB, LTB, sm.vt + 16 * Vt * LT, LT, lane, 16 * It + 16);
    store4(gU + ((size_t)(It * (D / 16) + Vt) * 64 + lane) * 4, acc[0], acc[1], acc[2], acc[3]);
  }
  }  // listed chunks
}

// ------------------------------------------------------------------ launchers
template <int D, int C, typename IO, typename E>
static hipError_t launch_exact_t(const PrepParams& p, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((kda_chunk_prep_exact_kernel<D, C, IO, E>), dim3(grid), dim3(kPrepThreads),
                     0, st, p);
  return hipGetLastError();
}

template <int D, typename IO, typename E>
static hipError_t launch_exact_c(const PrepParams& p, int C, unsigned grid, hipStream_t st) {
  switch (C) {
    case 16: return launch_exact_t<D, 16, IO, E>(p, grid, st);
    case 32: return launch_exact_t<D, 32, IO, E>(p, grid, st);
    case 64:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_exact_t<D, 64, IO, E>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO, typename E>
static hipError_t launch_exact_d(const PrepParams& p, int D, int C, unsigned grid, hipStream_t st) {
  switch (D) {
    case 16: return launch_exact_c<16, IO, E>(p, C, grid, st);
    case 32: return launch_exact_c<32, IO, E>(p, C, grid, st);
    case 64: return launch_exact_c<64, IO, E>(p, C, grid, st);
    case 128: return launch_exact_c<128, IO, E>(p, C, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prep_exact(const PrepParams& p, int D, int C, bool fp32, unsigned grid,
                             hipStream_t st) {
  return fp32 ? launch_exact_d<float, float>(p, D, C, grid, st)
              : launch_exact_d<__bf16, __bf16>(p, D, C, grid, st);
}

}  // namespace kda
