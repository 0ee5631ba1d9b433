// Chunk preparation for the KDA prefill: one workgroup per (sequence, head,
// chunk of C tokens).  Everything here is independent across chunks; the serial
// dependence on the state is left to the state walk.
//
// Per chunk (Gamma = chunk-local cumulative sum of the log-decay g, per channel;
// Lambda = exp(Gamma); all decays act on the key channels):
//   1. short conv + SiLU + L2 norm of q, k (and conv + SiLU of v)
//   2. Gamma, Lambda, the chunk decay Lambda_C
//   3. A_ij = beta_i sum_c k_ic k_jc exp(Gamma_ic - Gamma_jc)   (j < i)
//      P_ij = scale * sum_c q_ic k_jc exp(Gamma_ic - Gamma_jc)  (j <= i)
//   4. T = (I + A)^-1 (unit lower triangular)
//   5. W = T diag(beta) (K * Lambda),  U~ = T diag(beta) V
// The triangular structure is the WY/UT form of the product of the generalised
// Householder factors (I - beta k k^T) that the delta rule composes.
//
// Step 3 as matrix products over 16-token blocks, per channel: with G_p the
// cumulative decay just before block p, s_p = G_p - G_{p+1} its span and
// m_p = (G_p + G_{p+1}) / 2 the middle of the block's range,
//   a_i = exp(Gamma_i - m_p) for i in block p,   b_j = exp(m_q - Gamma_j) for j in block q,
//   exp(Gamma_i - Gamma_j) = a_i * exp(m_p - m_q) * b_j.
// a and b lie within exp(+-s/2), so every operand is representable in fp32/bf16
// while s stays below ~166 nats; a chunk with a wider block span is listed in the
// workspace and recomputed by the exact preparation kernel.  The pair factor of
// blocks p > q is exp(-(s_p + s_q)/2) or smaller and may underflow although the
// products it scales do not, so it is applied to the b side in two steps whose
// partial products stay representable:
//   b_j exp(-s_q/2) = exp(G_{q+1} - Gamma_j) <= 1,  then times exp(m_p - G_{q+1}) <= 1
// (both factors <= 1: a product underflows only where its true value does).
#include "kda_convnorm.h"
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

constexpr float kFatalSpan = 240.f * kLn2;  // widest block span factored (240 log2 units, ~166 nats)

// Threads per workgroup: 256 for bf16 (two workgroups share a compute unit, so
// one's loads overlap the other's arithmetic), 512 for fp32 (whose rows take
// twice the registers, so each thread holds half as many tokens).
template <typename E> constexpr int fast_threads() { return sizeof(E) == 2 ? 256 : 512; }

// Work split of the front end: each thread takes TOK consecutive tokens x 8
// channels of the chunk.
template <int D, int C, int NTH>
struct FastTile {
  static constexpr int NOCT = D / 8;  // 8-channel groups per token row
  static constexpr int TOK = C * NOCT / NTH > 0 ? C * NOCT / NTH : 1;
  static constexpr int NSEG = C / TOK;  // token segments
  static constexpr int ITEMS = NSEG * NOCT;
  static_assert(ITEMS <= NTH, "tile does not fit one pass");
  static_assert(16 % TOK == 0, "a segment stays inside one 16-token block");
};

template <int D, int C, typename E, int NSEG>
struct FastSmem {
  static constexpr int ES = (int)sizeof(E);
  static constexpr int PE = 16 / ES;               // 16-byte row padding, in elements
  static constexpr int LQ = D + PE;                // operand rows (k = channel)
  static constexpr int LT = C + PE;                // rows of T in E (k = token)
  static constexpr int LA = C + 4;                 // A and T rows (floats)
  static constexpr int NB = C / 16;                // 16-token blocks
  static constexpr int NPAIR = NB * (NB - 1) / 2 > 0 ? NB * (NB - 1) / 2 : 1;
  // One region, used in turn for
  //   the operand arrays [C][LQ]: RA = beta k a (rows i), RP = q a (rows i),
  //     CB = k b (rows j), with a, b the block-midpoint decay factors;
  //   A, T (float), the solve's scratch and T in E;
  //   (beta K Lambda)^T and (beta V)^T as swizzled [D][C] images, next to T in E.
  static constexpr int OPS = 3 * C * LQ * ES;
  static constexpr int SOLVE = (2 * C * LA + 4 * 16 * 17) * 4;
  static constexpr int IMGS = 2 * D * C * ES;
  static constexpr int KLT_OFF = 0;
  static constexpr int VT_OFF = D * C * ES;
  static constexpr int TB_OFF = ((SOLVE > IMGS ? SOLVE : IMGS) + 15) / 16 * 16;
  static constexpr int LAST = TB_OFF + C * LT * ES;
  static constexpr int R1 = OPS > LAST ? OPS : LAST;
  alignas(16) char r1[R1];
  alignas(16) float tot[NSEG * D];     // segment totals, then exclusive prefixes
  // per block p and channel, with G_p the cumulative decay (nats) before block p and
  // m_p = (G_p + G_{p+1}) / 2:
  alignas(16) float mid[NB * D];       // m_p times log2(e)
  alignas(16) float emid[NB * D];      // exp(m_p)
  alignas(16) float ecm[NB * D];       // exp(Gamma_C - m_p)
  alignas(16) float hs[NB * D];        // exp(-s_p / 2) = exp(G_{p+1} - m_p)
  alignas(16) float xf[NPAIR * D];     // exp(m_R - G_{Q+1}) for blocks R > Q
  alignas(16) float filt[3 * 4 * D];   // the head's conv filters [q, k, v][tap][D]
  int fatal;
};

__device__ __forceinline__ int pair_index(int R, int Q) {
  // pairs R > Q in the order (1,0), (2,0), (2,1), (3,0), ...
  return R * (R - 1) / 2 + Q;
}

// Multiply the operand fragment element-wise by a per-k factor f[k] (k = channel).
template <int K>
__device__ __forceinline__ void scale_k(RowFrag<__bf16, K>& fr, const float* f, int g) {
  using FR = RowFrag<__bf16, K>;
#pragma unroll
  for (int i = 0; i < FR::N; ++i)
#pragma unroll
    for (int e = 0; e < FR::PER; ++e)
      fr.v[i][e] = (__bf16)((float)fr.v[i][e] * f[i * FR::STEP + FR::PER * g + e]);
}
template <int K>
__device__ __forceinline__ void scale_k(RowFrag<float, K>& fr, const float* f, int g) {
#pragma unroll
  for (int i = 0; i < RowFrag<float, K>::N; ++i) fr.v[i] *= f[4 * i + g];
}

// Multiply the operand fragment element-wise by f1[k], then by f2[k] (two
// roundings in fp32, so a product of two tiny factors cannot underflow where the
// operand times f1 stays representable).
template <int K>
__device__ __forceinline__ void scale_k2(RowFrag<__bf16, K>& fr, const float* f1, const float* f2,
                                         int g) {
  using FR = RowFrag<__bf16, K>;
#pragma unroll
  for (int i = 0; i < FR::N; ++i)
#pragma unroll
    for (int e = 0; e < FR::PER; ++e) {
      const int k = i * FR::STEP + FR::PER * g + e;
      fr.v[i][e] = (__bf16)(((float)fr.v[i][e] * f1[k]) * f2[k]);
    }
}
template <int K>
__device__ __forceinline__ void scale_k2(RowFrag<float, K>& fr, const float* f1, const float* f2,
                                         int g) {
#pragma unroll
  for (int i = 0; i < RowFrag<float, K>::N; ++i) fr.v[i] = (fr.v[i] * f1[4 * i + g]) * f2[4 * i + g];
}

// Swizzled image of a [rows][C] matrix used as a matrix-core operand along its
// rows: 16-byte chunk c of row `row` sits at c ^ ((row ^ (row >> 3)) % RC).  Both
// the transposed stores that build it (consecutive rows 8 apart per lane group)
// and the fragment reads (16 consecutive rows) spread over the banks.
template <typename E, int C>
struct TImg {
  static constexpr int EPC = 16 / (int)sizeof(E);
  static constexpr int RC = C / EPC;
  __device__ __forceinline__ static int at(int row, int k) {
    return row * C + (((k / EPC) ^ ((row ^ (row >> 3)) & (RC - 1))) * EPC) + (k % EPC);
  }
};

template <int K, typename E>
__device__ __forceinline__ void load_timg(RowFrag<E, K>& f, const E* img, int row, int g) {
  using FR = RowFrag<E, K>;
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int i = 0; i < FR::N; ++i)
      f.v[i] = *reinterpret_cast<const typename FR::V*>(img + TImg<E, K>::at(row, i * FR::STEP + FR::PER * g));
  } else {
#pragma unroll
    for (int i = 0; i < FR::N; ++i) f.v[i] = img[TImg<E, K>::at(row, 4 * i + g)];
  }
}

// TOK consecutive elements of one image row (TOK * sizeof(E) <= 16 bytes, inside
// one 16-byte chunk)
template <int TOK, typename E>
__device__ __forceinline__ void store_run(E* dst, const E (&v)[TOK]) {
  if constexpr (TOK * sizeof(E) == 16) {
    typedef E run_t __attribute__((ext_vector_type(TOK)));
    run_t x;
#pragma unroll
    for (int i = 0; i < TOK; ++i) x[i] = v[i];
    *reinterpret_cast<run_t*>(dst) = x;
  } else if constexpr (TOK * sizeof(E) == 8 || TOK * sizeof(E) == 4) {
    typedef E run_t __attribute__((ext_vector_type(TOK)));
    run_t x;
#pragma unroll
    for (int i = 0; i < TOK; ++i) x[i] = v[i];
    *reinterpret_cast<run_t*>(dst) = x;
  } else {
#pragma unroll
    for (int i = 0; i < TOK; ++i) dst[i] = v[i];
  }
}

// One workgroup per (sequence, head, chunk).
template <int D, int C, typename IO, typename E>
__global__ __launch_bounds__(fast_threads<E>()) void kda_chunk_prep_kernel(PrepParams p) {
  constexpr int NTH = fast_threads<E>();
  using TL = FastTile<D, C, NTH>;
  constexpr int NOCT = TL::NOCT, TOK = TL::TOK, NSEG = TL::NSEG, ITEMS = TL::ITEMS;
  using SM = FastSmem<D, C, E, NSEG>;
  __shared__ SM sm;
  constexpr int LQ = SM::LQ, LT = SM::LT, LA = SM::LA, NB = SM::NB;
  constexpr int NW = NTH / 64;
  constexpr RecordLayout RL = record_layout(C, D, sizeof(E));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  // Chunk-major order: the workgroups running at the same time cover every head
  // of a few consecutive chunks, so together they read whole token rows of q, k,
  // v, g (all heads of a token are adjacent in memory), and write one
  // contiguous stretch of records (rec_slot: workgroup i is record slot i).
  // Packed sequences: slot gc of head h, a chunk of the sequence owning that
  // slot (slots past the last one in use have nothing to do).  b is the
  // sequence (conv state), tok0 its first token row, Tq its length.
  int n, h, b, rec, Tq;
  long tok0;
  if (p.seqs.bounds == nullptr) {
    const int BH = p.B * p.H;
    n = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    h = bh % p.H;
    b = bh / p.H;
    rec = (int)rec_slot(n, bh, BH);
    tok0 = (long)b * p.T;
    Tq = p.T;
  } else {
    const int gc = blockIdx.x / p.H;
    h = blockIdx.x % p.H;
    if (gc >= p.seqs.cstart[p.seqs.n_seqs]) return;
    b = seq_of_slot(p.seqs.cstart, p.seqs.n_seqs, gc);
    n = gc - p.seqs.cstart[b];
    tok0 = p.seqs.bounds[b];
    Tq = p.seqs.bounds[b + 1] - p.seqs.bounds[b];
    rec = (int)rec_slot(gc, h, p.H);
    if (n < 0 || (long)n * C >= Tq) return;  // inconsistent tables: touch nothing
  }
  const int t0 = (p.c0 + n) * C;  // first token of the chunk in its sequence
  char* recp = p.ws + (size_t)rec * RL.bytes;
  E* gW = reinterpret_cast<E*>(recp) + RL.w;
  E* gQL = reinterpret_cast<E*>(recp) + RL.ql;
  E* gKT = reinterpret_cast<E*>(recp) + RL.kt;
  E* gU = reinterpret_cast<E*>(recp) + RL.u;
  E* gP = reinterpret_cast<E*>(recp) + RL.p;
  float* gLC = reinterpret_cast<float*>(recp + RL.lc_bytes);
  E* RA = reinterpret_cast<E*>(sm.r1);
  E* RP = RA + C * LQ;
  E* CB = RP + C * LQ;

  // ---------------------------------------------------------------- phase 1
  const bool active = tid < ITEMS;
  const int s = active ? tid / NOCT : 0;  // token segment
  const int j = tid % NOCT;
  const int ch = 8 * j;
  const int pb = (TOK * s) / 16;          // 16-token block of this segment
  const int tf = t0 + TOK * s;
  // every global load of this phase is issued before the first wait: the head's
  // filters, the q/k/v windows, g and beta
  const bool conv = p.conv_w != nullptr;
  FilterRegs<D, NTH> fr;
  if (conv) load_filters<D, NTH>(p.conv_w, p.H, h, tid, fr);
  Raw8<IO> win[3][TOK + 3];
  const long HDl = (long)p.H * D;
  const IO* cs_in = p.conv_state_in == nullptr
                        ? nullptr
                        : static_cast<const IO*>(p.conv_state_in) + (long)b * 9 * HDl;
  front_load<TOK, IO>(static_cast<const IO*>(p.q) + tok0 * HDl,
                      static_cast<const IO*>(p.k) + tok0 * HDl,
                      static_cast<const IO*>(p.v) + tok0 * HDl, cs_in, conv, 0, Tq, p.H, D, h,
                      ch, t0, C, tf, win);
  // g rows and beta of tokens [t0, t0 + C): range-checked loads read zeros past
  // the end of the sequence
  Raw8<IO> graw[TOK];
  float braw[TOK];
  const int nt = Tq - t0 < C ? Tq - t0 : C;  // tokens of the sequence in this chunk
  // raw gate projection: this thread's 8 channel biases and minus the head's rate
  const bool gact = p.A_log != nullptr;
  f32x4 gb0 = {0.f, 0.f, 0.f, 0.f}, gb1 = gb0;
  float gneg = 0.f;
  if (gact) {
    const f32x4* bp = reinterpret_cast<const f32x4*>(p.dt_bias + (size_t)h * D + ch);
    gb0 = bp[0];
    gb1 = bp[1];
    gneg = -__expf(p.A_log[h]) * kLn2;  // softplus_log2 gives log2 units; the decay is kept in nats
  }
  {
    constexpr int ES = (int)sizeof(IO);
    const long HD = (long)p.H * D;
    const BufRes rg = make_buf(static_cast<const IO*>(p.g) + (tok0 + t0) * HD + (long)h * D,
                               (unsigned)(((long)(nt - 1) * HD + D) * ES));
    const BufRes rb = make_buf(static_cast<const IO*>(p.beta) + (tok0 + t0) * p.H + h,
                               (unsigned)(((long)(nt - 1) * p.H + 1) * ES));
    const int gv = (TOK * s) * (int)(HD * ES) + ch * ES;
    const int bv = (TOK * s) * p.H * ES;
#pragma unroll
    for (int m = 0; m < TOK; ++m) {
      graw[m].load(rg, gv + m * (int)(HD * ES), 0);
      if constexpr (ES == 2)
        braw[m] = __builtin_bit_cast(__bf16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(
                                                 rb, bv + m * p.H * ES, 0, 0));
      else
        braw[m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                rb, bv + m * p.H * ES, 0, 0));
    }
  }
  if (tid == 0) sm.fatal = 0;
  __builtin_amdgcn_sched_barrier(0);  // the loads above are all issued first
  if (conv) store_filters<D, NTH>(fr, sm.filt, tid, kLog2e);
  __syncthreads();  // filters are in LDS
  // filters times log2(e): q and k come out as they are, v times log2(e)
  float yq[TOK][8], yk[TOK][8], yv[TOK][8], qk[TOK];
  front_compute<TOK, D, IO, false, false, true>(win, sm.filt, conv, ch, tf, Tq, active, p.l2 != 0,
                                                p.eps, p.scale, yq, yk, yv, qk);
  const float vunit = conv ? kLn2 : 1.0f;
  // cumulative decay (nats) within the segment.  Past the end of the sequence g
  // and beta are 0 (the range-checked loads give zeros; the activations of raw
  // projections are masked there), which is all the later phases need of those
  // tokens.
  float gc[TOK][8], bt[TOK];
#pragma unroll
  for (int m = 0; m < TOK; ++m) {
    const bool in_seq = TOK * s + m < nt;
    bt[m] = p.beta_logits ? (in_seq ? sigmoid_fast(braw[m]) : 0.f) : braw[m];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float gv;  // nats
      if (gact)
        gv = in_seq ? gneg * softplus_log2(graw[m][c] + (c < 4 ? gb0[c] : gb1[c - 4])) : 0.f;
      else
        gv = graw[m][c];
      gc[m][c] = m == 0 ? gv : gc[m - 1][c] + gv;
    }
  }
  if (active) store8(sm.tot + s * D + ch, gc[TOK - 1]);
  __syncthreads();
  // one thread per channel: exclusive scan over segments, block boundaries,
  // midpoints and the pair factors
  if (tid < D) {
    const int c = tid;
    constexpr int SPB = 16 / TOK;  // segments per block
    float acc = 0.f;
    float gbl[NB + 1];
    gbl[0] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NSEG; ++s2) {
      const float v = sm.tot[s2 * D + c];
      sm.tot[s2 * D + c] = acc;
      acc += v;
      if ((s2 + 1) % SPB == 0) gbl[(s2 + 1) / SPB] = acc;
    }
    // exponentials in base 2 of log2(e) times the decays
    gLC[c] = __builtin_amdgcn_exp2f(acc * kLog2e);
    bool fatal = false;
    float md[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      md[q] = 0.5f * (gbl[q] + gbl[q + 1]);
      sm.mid[q * D + c] = md[q] * kLog2e;  // the operands use it in log2 units
      sm.emid[q * D + c] = __builtin_amdgcn_exp2f(md[q] * kLog2e);
      sm.ecm[q * D + c] = __builtin_amdgcn_exp2f((acc - md[q]) * kLog2e);
      sm.hs[q * D + c] = __builtin_amdgcn_exp2f((gbl[q + 1] - md[q]) * kLog2e);
      fatal |= gbl[q] - gbl[q + 1] > kFatalSpan;
    }
#pragma unroll
    for (int R = 1; R < NB; ++R)
#pragma unroll
      for (int Q = 0; Q < R; ++Q)
        sm.xf[pair_index(R, Q) * D + c] = __builtin_amdgcn_exp2f((md[R] - gbl[Q + 1]) * kLog2e);
    if (fatal) atomicOr(&sm.fatal, 1);
  }
  __syncthreads();
  if (p.y_out != nullptr && active) {
    // backward mode: the front end's outputs (record element type) and the
    // cumulative decay (float32)
    float pre[8];
    load8(&sm.tot[s * D + ch], pre);
    const long HD = (long)p.H * D;
    const long plane = (long)p.B * p.T * HD;
#pragma unroll
    for (int m = 0; m < TOK; ++m) {
      const int t = tf + m;
      if (t < Tq) {
        const long row = (tok0 + t) * HD + (long)h * D + ch;
        store8(static_cast<E*>(p.y_out) + row, yq[m]);
        store8(static_cast<E*>(p.y_out) + plane + row, yk[m]);
        float vv[8], gam[8];  // v as it is; the cumulative decay in log2 units
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          vv[c] = yv[m][c] * vunit;
          gam[c] = (gc[m][c] + pre[c]) * kLog2e;
        }
        store8(static_cast<E*>(p.y_out) + 2 * plane + row, vv);
        store8(p.gam_out + row, gam);
        if (j == 0) p.beta_out[(tok0 + t) * p.H + h] = bt[m];
      }
    }
  }
  if (sm.fatal) {
    // decays too strong for the factoring: the exact preparation redoes this chunk
    if (tid == 0) {
      const unsigned slot = atomicAdd(p.fb_count, 1u);
      p.fb_list[slot] = (unsigned)rec;
    }
    return;
  }
  // operands: with Gamma_i the cumulative decay and m the midpoint of token
  // i's block, a_i = exp(Gamma_i - m), b_i = exp(m - Gamma_i), and
  //   Lambda_i = a_i exp(m),   exp(Gamma_C - Gamma_i) = b_i exp(Gamma_C - m).
  // (Where exp(m) or exp(Gamma_C - m) underflows, the true value is below
  // exp(s/2) times that, far under the rounding of the other terms.)
  E kv[2][8][TOK];  // beta K Lambda and beta V, kept for the transposed images
  if (active) {
    float pre[8], md[8], em[8], ec[8];
    load8(&sm.tot[s * D + ch], pre);
    load8(&sm.mid[pb * D + ch], md);
    load8(&sm.emid[pb * D + ch], em);
    load8(&sm.ecm[pb * D + ch], ec);
    float kt[8][TOK];
#pragma unroll
    for (int m = 0; m < TOK; ++m) {
      const int tl = TOK * s + m;
      const float btv = bt[m] * vunit;
      float ra[8], rp[8], cb[8], ql[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float gam = gc[m][c] + pre[c];  // nats; md is in log2 units
        const float a = __builtin_amdgcn_exp2f(fmaf(gam, kLog2e, -md[c]));
        const float bb = __builtin_amdgcn_exp2f(fmaf(-gam, kLog2e, md[c]));
        const float lam = a * em[c];
        const float bk = bt[m] * yk[m][c];
        ra[c] = bk * a;
        rp[c] = yq[m][c] * a;
        cb[c] = yk[m][c] * bb;
        ql[c] = yq[m][c] * lam;
        kt[c][m] = yk[m][c] * (bb * ec[c]);
        kv[0][c][m] = from_f32<E>(bk * lam);
        kv[1][c][m] = from_f32<E>(btv * yv[m][c]);
      }
      store8(RA + tl * LQ + ch, ra);
      store8(RP + tl * LQ + ch, rp);
      store8(CB + tl * LQ + ch, cb);
      store8(gQL + (size_t)tl * D + ch, ql);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      E run[TOK];
#pragma unroll
      for (int m = 0; m < TOK; ++m) run[m] = from_f32<E>(kt[c][m]);
      store_run<TOK>(gKT + (size_t)(ch + c) * C + TOK * s, run);
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- phase 2
  // A^T / P^T tiles (rows j, columns i) of the lower block triangle, round robin
  // over waves; for blocks R > Q the k b rows take the pair factor.  Channels go
  // in pieces of KC (fp32 fragments take four times the registers).
  constexpr int NTILE = NB * (NB + 1) / 2;
  constexpr int TPW = (NTILE + NW - 1) / NW;
  constexpr int KC = sizeof(E) == 2 ? D : (D < 32 ? D : 32);
  f32x4 accA[TPW], accP[TPW];
  int tR[TPW], tQ[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    int idx = wave + NW * i, R = 0;
    while (idx > R) { idx -= R + 1; ++R; }
    tR[i] = (wave + NW * i < NTILE) ? R : -1;
    tQ[i] = idx;
    accA[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    accP[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (tR[i] < 0) continue;
    const int R0 = tR[i], Q0 = tQ[i];
#pragma unroll
    for (int kc = 0; kc < D; kc += KC) {
      RowFrag<E, KC> cf, fa, fp;
      cf.load(CB + (16 * Q0 + r) * LQ + kc, g4);
      if (R0 != Q0) scale_k2<KC>(cf, &sm.hs[Q0 * D + kc], &sm.xf[pair_index(R0, Q0) * D + kc], g4);
      fa.load(RA + (16 * R0 + r) * LQ + kc, g4);
      fp.load(RP + (16 * R0 + r) * LQ + kc, g4);
      mma<KC>(accA[i], cf, fa);
      mma<KC>(accP[i], cf, fp);
    }
  }
  __syncthreads();  // the operands are dead

  // ---------------------------------------------------------------- phase 3
  float* sA = reinterpret_cast<float*>(sm.r1);  // [C][LA]
  float* sT = sA + C * LA;                      // [C][LA]: the lower block triangle of T
  float* scr = sT + C * LA;                     // [4][16][17]
  // T in the matrix-core element type, after A / T / scratch, written by the solve
  // as it goes.  The causal k-steps of the W, U~ products read row tile It up to
  // column ceil(16 (It + 1) / STEPC) STEPC: the part of that beyond the diagonal
  // block is zero.
  E* tb = reinterpret_cast<E*>(sm.r1 + SM::TB_OFF);
  {
    constexpr int STEPC = RowFrag<E, C>::STEP;
    for (int It = 0; It < NB; ++It) {
      const int c0 = 16 * (It + 1);
      const int ce0 = (c0 + STEPC - 1) / STEPC * STEPC;
      const int ce = ce0 < C ? ce0 : C;
      const int w = ce - c0;  // columns to clear in each of the tile's 16 rows
      for (int it = tid; it < 16 * w; it += NTH)
        tb[(16 * It + it / w) * LT + c0 + it % w] = from_f32<E>(0.f);
    }
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int R = tR[i], Q = tQ[i];
    if (R < 0) continue;
    const int ii = 16 * R + r;
    const int jj = 16 * Q + 4 * g4;
    float av[4], pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool lowA = (R != Q) || (jj + e < ii);
      const bool lowP = (R != Q) || (jj + e <= ii);
      av[e] = lowA ? accA[i][e] : 0.f;
      pv[e] = lowP ? accP[i][e] : 0.f;
    }
    *reinterpret_cast<f32x4*>(&sA[ii * LA + jj]) = f32x4{av[0], av[1], av[2], av[3]};
    store4(gP + (size_t)ii * C + jj, pv[0], pv[1], pv[2], pv[3]);
  }
  __syncthreads();

  // ---------------------------------------------------------------- phase 4
  // T = (I + A)^-1: diagonal 16x16 blocks by forward substitution, one column
  // per thread
  if (tid < C) {
    const int pq = tid >> 4, col = tid & 15;
    const float* Ab = sA + (16 * pq) * LA + 16 * pq;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < i; ++jj) acc = fmaf(-Ab[i * LA + jj], x[jj], acc);
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sT[(16 * pq + i) * LA + 16 * pq + col] = x[i];
      tb[(16 * pq + i) * LT + 16 * pq + col] = from_f32<E>(x[i]);
    }
  }
  __syncthreads();
  // off-diagonal blocks, block row by block row (wave qb computes block column qb):
  //   T_pq = -T_pp * sum_{r=q}^{p-1} A_pr T_rq
  static_assert(NB - 1 <= NW, "a wave per block column");
  for (int pr = 1; pr < NB; ++pr) {
    const int qb = wave;
    float* xs = scr + (wave & 3) * 16 * 17;
    if (qb < pr) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int rb = qb; rb < pr; ++rb) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float a = sA[(16 * pr + r) * LA + 16 * rb + k0 + g4];
          const float bv = sT[(16 * rb + k0 + g4) * LA + 16 * qb + r];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[(4 * g4 + e) * 17 + r] = acc[e];
    }
    __syncthreads();
    if (qb < pr) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const float a = sT[(16 * pr + r) * LA + 16 * pr + k0 + g4];
        const float bv = xs[(k0 + g4) * 17 + r];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sT[(16 * pr + 4 * g4 + e) * LA + 16 * qb + r] = -acc[e];
        tb[(16 * pr + 4 * g4 + e) * LT + 16 * qb + r] = from_f32<E>(-acc[e]);
      }
    }
    __syncthreads();
  }
  if (p.t_out != nullptr) {
    // backward mode: T^T in the element type (the upper triangle of T is not
    // computed here)
    E* to = static_cast<E*>(p.t_out) + (size_t)rec * C * C;
    for (int it = tid; it < C * C; it += NTH) {
      const int jj = it / C, i = it % C;  // to[jj][i] = T[i][jj]
      to[it] = from_f32<E>(jj <= i ? sT[i * LA + jj] : 0.f);
    }
  }
  __syncthreads();  // A and T (float) are dead

  // ---------------------------------------------------------------- phase 5
  // (beta K Lambda)^T and (beta V)^T as swizzled [D][C] images
  E* klt = reinterpret_cast<E*>(sm.r1 + SM::KLT_OFF);
  E* vt = reinterpret_cast<E*>(sm.r1 + SM::VT_OFF);
  static_assert(SM::IMGS <= SM::TB_OFF, "transposed images stay clear of T");
  if (active) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int at = TImg<E, C>::at(ch + c, TOK * s);
      store_run<TOK>(klt + at, kv[0][c]);
      store_run<TOK>(vt + at, kv[1][c]);
    }
  }
  __syncthreads();
  // W^T tiles (c, i) = (beta K Lambda)^T T^T and U~ tiles (i, v) = T (beta V): the
  // NW / NB waves of token tile It split its 2 D/16 tiles; the T rows of the
  // token tile are loaded once per wave, and the causal k-steps stop at the
  // tile's diagonal
  constexpr int STEPC = RowFrag<E, C>::STEP;
  constexpr int WPI = NW / NB;        // waves per token tile
  constexpr int DT = D / 16;          // channel (or value) tiles
  static_assert(NW % NB == 0, "waves split evenly over the token tiles");
  {
    const int It = wave % NB, sub = wave / NB;
    const int steps = (16 * It + 16 + STEPC - 1) / STEPC;
    RowFrag<E, C> ft;
    ft.load(tb + (16 * It + r) * LT, g4);
    E* wrow = gW + (size_t)(16 * It + r) * D + 4 * g4;
#pragma unroll
    for (int q = 0; q < (DT + WPI - 1) / WPI; ++q) {
      const int Ct = sub + WPI * q;
      if (DT % WPI == 0 || Ct < DT) {
        RowFrag<E, C> fa;
        load_timg<C>(fa, klt, 16 * Ct + r, g4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mma<C>(acc, fa, ft, steps);
        store4(wrow + 16 * Ct, acc[0], acc[1], acc[2], acc[3]);
      }
    }
    E* urow = gU + ((size_t)It * DT * 64 + lane) * 4;
#pragma unroll
    for (int q = 0; q < (DT + WPI - 1) / WPI; ++q) {
      const int Vt = sub + WPI * q;
      if (DT % WPI == 0 || Vt < DT) {
        RowFrag<E, C> fb;
        load_timg<C>(fb, vt, 16 * Vt + r, g4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mma<C>(acc, ft, fb, steps);
        store4(urow + (size_t)Vt * 64 * 4, acc[0], acc[1], acc[2], acc[3]);
      }
    }
  }
}

// ------------------------------------------------------------ conv_norm alone
// tokens per thread of the standalone front end (fp32 rows take twice the registers)
template <typename IO> constexpr int conv_norm_tokens() { return sizeof(IO) == 2 ? 4 : 2; }

template <int D, typename IO>
__global__ __launch_bounds__(256) void kda_conv_norm_kernel(ConvNormParams p) {
  constexpr int NOCT = D / 8;
  constexpr int TT = conv_norm_tokens<IO>();
  constexpr int TOK = 256 / NOCT * TT;  // tokens per workgroup
  __shared__ alignas(16) float filt[3 * 4 * D];
  const int tid = threadIdx.x;
  const int nblk = (p.T + TOK - 1) / TOK;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int h = bh % p.H, b = bh / p.H;
  const int s = tid / NOCT, j = tid % NOCT;
  const int tf = blk * TOK + TT * s;
  const bool active = tf < p.T;
  FilterRegs<D, 256> fr;
  load_filters<D, 256>(p.conv_w, p.H, h, tid, fr);
  Raw8<IO> win[3][TT + 3];
  front_load<TT, IO>(static_cast<const IO*>(p.q), static_cast<const IO*>(p.k),
                     static_cast<const IO*>(p.v), static_cast<const IO*>(p.conv_state_in), true, b,
                     p.T, p.H, D, h, 8 * j, blk * TOK, TOK, tf, win);
  __builtin_amdgcn_sched_barrier(0);
  store_filters<D, 256>(fr, filt, tid);
  __syncthreads();  // filters are in LDS
  float yq[TT][8], yk[TT][8], yv[TT][8], qk[TT];
  front_compute<TT, D, IO>(win, filt, true, 8 * j, tf, p.T, active, p.l2 != 0, p.eps, 1.0f, yq,
                           yk, yv, qk);
  if (!active) return;
  const size_t HD = (size_t)p.H * D;
  IO* oq = static_cast<IO*>(p.q_out);
  IO* ok = static_cast<IO*>(p.k_out);
  IO* ov = static_cast<IO*>(p.v_out);
#pragma unroll
  for (int m = 0; m < TT; ++m) {
    const int t = tf + m;
    if (t >= p.T) break;
    const size_t off = ((size_t)b * p.T + t) * HD + (size_t)h * D + 8 * j;
    store8(oq + off, yq[m]);
    store8(ok + off, yk[m]);
    store8(ov + off, yv[m]);
  }
}

// --------------------------------------------------------- conv state hand-over
// conv_state_out[b][i][tau][c] = raw input at position T - 3 + tau (tau = 0..2)
// of sequence b, taken from the previous state when that position is < 0 (T the
// sequence's length; packed sequences read their bounds).  Each thread reads its
// three values before writing them, so out may equal in.
template <typename IO>
__global__ __launch_bounds__(256) void kda_conv_tail_kernel(TailParams p) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.B * 3 * p.HD;
  if (idx >= total) return;
  const int c = (int)(idx % p.HD);
  const int i = (int)((idx / p.HD) % 3);
  const int b = (int)(idx / ((size_t)3 * p.HD));
  const IO* x = static_cast<const IO*>(p.x[i]);
  const IO* in = static_cast<const IO*>(p.conv_state_in);
  IO* out = static_cast<IO*>(p.conv_state_out);
  const long tok0 = p.bounds == nullptr ? (long)b * p.T : p.bounds[b];
  const int Tq = p.bounds == nullptr ? p.T : p.bounds[b + 1] - p.bounds[b];
  IO val[3];
#pragma unroll
  for (int tau = 0; tau < 3; ++tau) {
    const int t = Tq - 3 + tau;
    if (t >= 0)
      val[tau] = x[((size_t)tok0 + t) * p.HD + c];
    else if (in != nullptr)
      val[tau] = in[(((size_t)b * 3 + i) * 3 + (3 + t)) * p.HD + c];
    else
      val[tau] = from_f32<IO>(0.f);
  }
#pragma unroll
  for (int tau = 0; tau < 3; ++tau) out[(((size_t)b * 3 + i) * 3 + tau) * p.HD + c] = val[tau];
}

// ------------------------------------------------------ packed-sequence tables
// Inclusive scan over the 1024 threads of a workgroup (max or sum); red holds 16
// ints of scratch.  Every thread must call it.
template <bool ADD>
__device__ __forceinline__ int block_scan(int x, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x = ADD ? x + y : (y > x ? y : x);
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? red[lane] : (ADD ? 0 : -2147483647 - 1);
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(w, d, 64);
      if (lane >= d) w = ADD ? w + y : (y > w ? y : w);
    }
    if (lane < 16) red[lane] = w;
  }
  __syncthreads();
  if (wave > 0) {
    const int pre = red[wave - 1];
    x = ADD ? x + pre : (pre > x ? pre : x);
  }
  __syncthreads();  // red may be reused
  return x;
}

// Token bounds of the packed sequences, the running maximum of the caller's
// offsets clamped to [0, T] (so malformed offsets can only give empty or
// shortened sequences, never an access outside the tensors), and each sequence's
// first chunk slot, the exclusive running sum of its chunk count (cstart[n_seqs]
// = slots in use); optionally the same for blocks of FB tokens (fstart).  One
// workgroup of 1024 threads, n_seqs + 1 entries in blocks.
__global__ __launch_bounds__(1024) void kda_seq_index_kernel(IndexParams p) {
  __shared__ int red[16];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base <= p.n_seqs; base += 1024) {
    const int i = base + tid;
    int x = 0;
    if (i <= p.n_seqs) {
      x = p.cu_seqlens[i];
      x = x < 0 ? 0 : (x > p.T ? p.T : x);
    }
    x = block_scan<false>(x, red);
    if (x < carry) x = carry;
    if (i <= p.n_seqs) p.bounds[i] = x;
    __syncthreads();  // every thread has read carry
    if (tid == 1023) carry = x;
    __syncthreads();
  }
  // bounds are visible to the whole workgroup after the barrier above
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base <= p.n_seqs; base += 1024) {
    const int i = base + tid;
    const int cnt = i < p.n_seqs ? (p.bounds[i + 1] - p.bounds[i] + p.C - 1) / p.C : 0;
    const int incl = block_scan<true>(cnt, red) + carry;
    if (i <= p.n_seqs) p.cstart[i] = incl - cnt;
    __syncthreads();
    if (tid == 1023) carry = incl;
    __syncthreads();
  }
  if (p.fstart == nullptr) return;
  // the same for blocks of FB tokens
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base <= p.n_seqs; base += 1024) {
    const int i = base + tid;
    const int cnt = i < p.n_seqs ? (p.bounds[i + 1] - p.bounds[i] + p.FB - 1) / p.FB : 0;
    const int incl = block_scan<true>(cnt, red) + carry;
    if (i <= p.n_seqs) p.fstart[i] = incl - cnt;
    __syncthreads();
    if (tid == 1023) carry = incl;
    __syncthreads();
  }
}

// S_T = S0 (or zeros) for empty sequences.
__global__ __launch_bounds__(256) void kda_copy_state_kernel(const float* src, float* dst,
                                                             size_t n) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) dst[idx] = src ? src[idx] : 0.f;
}

// Clears the count of chunks handed to the exact preparation.
__global__ void kda_reset_count_kernel(unsigned* count) {
  if (threadIdx.x == 0) *count = 0u;
}

// ------------------------------------------------------------------ launchers
template <int D, int C, typename IO, typename E>
static hipError_t launch_prep_t(const PrepParams& p, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)p.B * p.H * p.nchunk);
  hipLaunchKernelGGL((kda_chunk_prep_kernel<D, C, IO, E>), dim3(grid), dim3(fast_threads<E>()), 0,
                     st, p);
  return hipGetLastError();
}

template <int D, typename IO, typename E>
static hipError_t launch_prep_c(const PrepParams& p, int C, hipStream_t st) {
  switch (C) {
    case 16: return launch_prep_t<D, 16, IO, E>(p, st);
    case 32: return launch_prep_t<D, 32, IO, E>(p, st);
    case 64:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_prep_t<D, 64, IO, E>(p, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO, typename E>
static hipError_t launch_prep_d(const PrepParams& p, int D, int C, hipStream_t st) {
  switch (D) {
    case 16: return launch_prep_c<16, IO, E>(p, C, st);
    case 32: return launch_prep_c<32, IO, E>(p, C, st);
    case 64: return launch_prep_c<64, IO, E>(p, C, st);
    case 128: return launch_prep_c<128, IO, E>(p, C, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prep(const PrepParams& p, int D, int C, bool fp32, hipStream_t st) {
  hipLaunchKernelGGL(kda_reset_count_kernel, dim3(1), dim3(64), 0, st, p.fb_count);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const hipError_t e = fp32 ? launch_prep_d<float, float>(p, D, C, st)
                            : launch_prep_d<__bf16, __bf16>(p, D, C, st);
  if (e != hipSuccess) return e;
  // the exact preparation of the listed chunks (exits at once when none is listed)
  const size_t nrec = (size_t)p.B * p.H * p.NT;
  const unsigned grid = (unsigned)(nrec < 512 ? nrec : 512);
  return launch_prep_exact(p, D, C, fp32, grid, st);
}

template <int D, typename IO>
static hipError_t launch_conv_norm_t(const ConvNormParams& p, hipStream_t st) {
  constexpr int TOK = 256 / (D / 8) * conv_norm_tokens<IO>();
  const int nblk = (p.T + TOK - 1) / TOK;
  const unsigned grid = (unsigned)((size_t)p.B * p.H * nblk);
  hipLaunchKernelGGL((kda_conv_norm_kernel<D, IO>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_conv_norm(const ConvNormParams& p, int D, bool fp32, hipStream_t st) {
  if (fp32) {
    switch (D) {
      case 16: return launch_conv_norm_t<16, float>(p, st);
      case 32: return launch_conv_norm_t<32, float>(p, st);
      case 64: return launch_conv_norm_t<64, float>(p, st);
      case 128: return launch_conv_norm_t<128, float>(p, st);
    }
  } else {
    switch (D) {
      case 16: return launch_conv_norm_t<16, __bf16>(p, st);
      case 32: return launch_conv_norm_t<32, __bf16>(p, st);
      case 64: return launch_conv_norm_t<64, __bf16>(p, st);
      case 128: return launch_conv_norm_t<128, __bf16>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv_tail(const TailParams& p, bool fp32, hipStream_t st) {
  const size_t total = (size_t)p.B * 3 * p.HD;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (fp32)
    hipLaunchKernelGGL((kda_conv_tail_kernel<float>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((kda_conv_tail_kernel<__bf16>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_seq_index(const IndexParams& p, hipStream_t st) {
  hipLaunchKernelGGL(kda_seq_index_kernel, dim3(1), dim3(1024), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(kda_copy_state_kernel, dim3(grid), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

}  // namespace kda
