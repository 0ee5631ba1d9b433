// Backward pass of the KDA prefill: the gradients of L = <o, dO> + <S_T, dS_T>
// with respect to the raw q, k, v, the log-decay g, beta, S0 and the conv filters
// and history.
//
// The forward is recomputed by the forward kernels in backward mode (chunk
// records, the front end's outputs, T^T per chunk, and the state at every chunk
// start).  With, per chunk (Gamma the chunk-local cumulative log-decay, Lambda =
// exp(Gamma), C tokens):
//   A_ij = beta_i sum_c k_ic k_jc exp(Gamma_ic - Gamma_jc) (j < i),  T = (I + A)^-1
//   Bk = diag(beta) (K * Lambda),  Bv = diag(beta) V,  W = T Bk,  U~ = T Bv
//   QL = Q' * Lambda (Q' = scale * q_hat),  P_ij = sum_c Q'_ic k_jc exp(Gamma_ic - Gamma_jc) (j <= i)
//   Ktil = K * exp(Gamma_C - Gamma),  LC = exp(Gamma_C)
//   U = U~ - W S,  O = QL S + P U,  S' = Diag(LC) S + Ktil^T U
// the backward is
//   reverse walk:  dU = P^T dO + Ktil dS',   dS = Diag(LC) dS' + QL^T dO - W^T dU
//   per chunk:     dQL = dO S^T,  dW = -dU S^T,  dKtil = U dS'^T,  dP = (dO U^T) on j <= i,
//                  dLC = rowsum(dS' * S),  dT = dW Bk^T + dU Bv^T,  dA = -T^T dT T^T (j < i),
//                  dBk = T^T dW,  dBv = T^T dU
// then the element terms and the pair terms of A and P (exp(Gamma_i - Gamma_j)
// evaluated per pair, never split), dGamma to dg by a reverse running sum over the
// chunk, and finally the front end in reverse (L2 norm, SiLU, convolution).
#include "kda_convnorm.h"
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {

// Tokens of record `rec`: `tok` is the token row of its first token (rows of the
// [rows of tokens][H][D] tensors are tok + t), `nval` how many of its C tokens
// exist (0 for an unused slot of a packed batch), h its head.  B equal-length
// sequences: rec = rec_slot(n, b H + h, B H).  Packed: rec = rec_slot(slot, h,
// H), the slot a chunk of the sequence that owns it (the workspace tables).
struct RecTok {
  long tok;
  int nval, h;
};
__device__ __forceinline__ RecTok rec_tokens(int rec, int B, int T, int H, int C, const SeqTables& sq) {
  RecTok g;
  if (sq.bounds == nullptr) {
    const int n = rec / (B * H), bh = rec % (B * H);
    g.h = bh % H;
    g.tok = (long)(bh / H) * T + (long)n * C;
    const int rem = T - n * C;
    g.nval = rem < C ? (rem > 0 ? rem : 0) : C;
  } else {
    const int slot = rec / H;
    g.h = rec % H;
    g.tok = 0;
    g.nval = 0;
    if (slot < sq.cstart[sq.n_seqs]) {
      const int sq_i = seq_of_slot(sq.cstart, sq.n_seqs, slot);
      const int n = slot - sq.cstart[sq_i];
      const int rem = sq.bounds[sq_i + 1] - sq.bounds[sq_i] - n * C;
      g.tok = sq.bounds[sq_i] + (long)n * C;
      g.nval = rem < C ? (rem > 0 ? rem : 0) : C;
    }
  }
  return g;
}

// ----------------------------------------------------------------- reverse walk
// The part of a forward record the reverse walk reads, as an LDS image (byte
// offsets): W [C][D], QL [C][D], KT [D][C], P [C][C] (swizzled as in the
// forward walk), LC [D] float.
template <int D, int C, typename E>
struct BwdImage {
  static constexpr int ES = (int)sizeof(E);
  static constexpr int W = 0;
  static constexpr int QL = W + C * D * ES;
  static constexpr int KT = QL + C * D * ES;
  static constexpr int P = KT + D * C * ES;
  static constexpr int LC = P + C * C * ES;
  static constexpr int BYTES = LC + D * 4;
  static constexpr int CHUNKS = BYTES / 16;
  static_assert(BYTES % 16 == 0, "whole 16-byte chunks");
};

// One workgroup per (sequence b, h, block of VB value columns); the D x VB block
// of dS stays in matrix-core accumulators, walking the sequence's chunks from the
// last to the first.  Per chunk, in the NT products C[i][j] = sum_k A[i][k] B[j][k]:
//   dU (t, v):  A = P^T rows t (P's column t, k = j >= t), B = dO^T rows v;
//               + A = Ktil rows t (KT's column t, k = c),  B = dS'^T rows v
//   dS (c, v):  A = QL^T rows c (QL's column c, k = t),   B = dO^T rows v;
//               - A = W^T rows c,                         B = dU^T rows v
// Split walk (p.nseg > 1): one workgroup per (sequence, head, segment, value
// block) walking the segment's chunks from the gradient of its end state in
// p.starts; only segment 0 writes dS0.  MAPW: the segments' reverse maps
// instead, for segments 1 .. nseg - 1: the walk from a zero end gradient (from
// dS_T for the last segment) with nothing stored per chunk, its result (the
// gradient of the segment's start state) written to the N slot of segment s - 1.
template <int D, int C, int VB, typename IO, typename E, int NT, bool MAPW>
__global__ __launch_bounds__(NT, 1) void kda_bwd_walk_kernel(BwdWalkParams p) {
  constexpr int NW = NT / 64;
  constexpr int PE = 16 / (int)sizeof(E);
  constexpr int ES = (int)sizeof(E);
  constexpr int LS = D + PE;  // sS rows: value column v, k = key channel c
  constexpr int LU = C + PE;  // sDU / sDO rows: value column v, k = token t
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
  using IMG = BwdImage<D, C, E>;
  __shared__ __attribute__((aligned(16))) char img[IMG::BYTES];
  __shared__ __attribute__((aligned(16))) E sS[VB * LS];
  __shared__ __attribute__((aligned(16))) E sDU[VB * LU];
  __shared__ __attribute__((aligned(16))) E sDO[2][VB * LU];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  // The value blocks of one (sequence, head) read the same records: they go to
  // the same XCD (workgroups are dealt round robin over the 8 XCDs), so the
  // second read of a record is served by that XCD's L2.
  const int total = p.B * p.H * NV;
  int bh, vblk, seg = 0;
  if (p.nseg > 1) {
    // (head, segment) groups of NV workgroups, numbered XCD by XCD
    const int grp = xcd_major(blockIdx.x, gridDim.x);
    vblk = grp % NV;
    bh = grp / NV % (p.B * p.H);
    seg = grp / NV / (p.B * p.H) + (MAPW ? 1 : 0);
  } else if (total % (8 * NV) == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    vblk = slot % NV;
    bh = (slot / NV) * 8 + xcd;
  } else {
    vblk = blockIdx.x % NV;
    bh = blockIdx.x / NV;
  }
  const int h = bh % p.H, b = bh / p.H;
  const int vb0 = vblk * VB;
  const size_t HD = (size_t)p.H * D;
  // the sequence's records (chunk n is record rec0 + n rstride, rec_slot), first
  // token row and length
  size_t rstride = (size_t)p.B * p.H;
  size_t rec0 = bh;
  long tok0 = (long)b * p.T;
  int Tq = p.T, nch = p.NT;
  if (p.seqs.bounds != nullptr) {
    const int c0 = p.seqs.cstart[b];
    tok0 = p.seqs.bounds[b];
    Tq = p.seqs.bounds[b + 1] - p.seqs.bounds[b];
    nch = (Tq + C - 1) / C;
    if (c0 + nch > p.NT) nch = c0 < p.NT ? p.NT - c0 : 0;  // inconsistent tables: stay in the head's slots
    rstride = (size_t)p.H;
    rec0 = rec_slot(c0, h, rstride);
  }
  // this workgroup's chunks [n_lo, n_hi) of the sequence
  int n_lo = 0, n_hi = nch;
  if (p.nseg > 1) {
    n_lo = seg * p.seg_len;
    n_hi = n_lo + p.seg_len < nch ? n_lo + p.seg_len : nch;
  }

  const int R = wave % RT;
  const bool has_u = FULL_U || wave < RT * VT;
  const int t_row = 16 * R + r;  // row of dU (token) this lane's A fragments hold

  // ---- copy of a record's image (the same source offsets for every chunk)
  constexpr int ITERS = (IMG::CHUNKS + NT - 1) / NT;
  uint32_t src_off[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    constexpr int RCD = D * ES / 16;
    constexpr int RCC = C * ES / 16;
    const int idx = it * NT + tid;
    const int byte = idx * 16;
    size_t off;
    if (byte < IMG::KT) {
      const bool isql = byte >= IMG::QL;
      const int ci = idx - (isql ? IMG::QL / 16 : 0);
      const int row = ci / RCD, cs = ci % RCD;
      off = (size_t)(isql ? RL.ql : RL.w) * ES + (size_t)(row * RCD + (cs ^ (row & (RCD - 1)))) * 16;
    } else if (byte < IMG::LC) {
      const bool isp = byte >= IMG::P;
      const int ci = idx - (isp ? IMG::P : IMG::KT) / 16;
      const int row = ci / RCC, cs = ci % RCC;
      off = (size_t)(isp ? RL.p : RL.kt) * ES + (size_t)(row * RCC + (cs ^ (row & (RCC - 1)))) * 16;
    } else {
      off = RL.lc_bytes + (size_t)(idx - IMG::LC / 16) * 16;
    }
    src_off[it] = (uint32_t)off;
  }
  auto issue_copy = [&](int n) {
    const char* recp = p.ws + (rec0 + n * rstride) * RL.bytes;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      if (it * NT + tid < IMG::CHUNKS)
        __builtin_amdgcn_global_load_lds(
            (const glb_void_t*)(recp + src_off[it]),
            (lds_void_t*)(img + (size_t)(it * NT + 64 * wave) * 16), 16, 0, 0);
    }
  };

  // ---- dO of a chunk: 8 consecutive value columns of one token per piece
  constexpr int DOP = C * VB / 8;                // pieces per chunk
  constexpr int DOIT = (DOP + NT - 1) / NT;
  Raw8<IO> dor[DOIT];
  auto load_do = [&](int n) {
#pragma unroll
    for (int it = 0; it < DOIT; ++it) {
      const int idx = it * NT + tid;
      const int tt = idx / (VB / 8), v8 = idx % (VB / 8);
      const int t = n * C + tt;
      if (idx < DOP && t < Tq)
        dor[it].load(static_cast<const IO*>(p.dO) + ((size_t)tok0 + t) * HD + (size_t)h * D + vb0 +
                     8 * v8);
      else
        dor[it] = Raw8<IO>{};
    }
  };
  auto stage_do = [&](int n) {
    E* dst = sDO[n & 1];
#pragma unroll
    for (int it = 0; it < DOIT; ++it) {
      const int idx = it * NT + tid;
      if (idx < DOP) {
        const int tt = idx / (VB / 8), v8 = idx % (VB / 8);
#pragma unroll
        for (int m = 0; m < 8; ++m) dst[(8 * v8 + m) * LU + tt] = from_f32<E>(dor[it][m]);
      }
    }
  };

  // ---- dS: initial value dS_T (or zero; a segment's from the composed
  // gradients), staged to LDS as the B operand
  f32x4 accS[NS];
  const size_t sbase = (size_t)bh * D * D;
  const float* g_in = p.dS_T != nullptr ? p.dS_T + sbase : nullptr;
  if (p.nseg > 1) {
    if constexpr (MAPW) g_in = seg == p.nseg - 1 ? g_in : nullptr;
    else g_in = p.starts + ((size_t)bh * p.nseg + seg) * D * D;
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = wave + NW * i;
    accS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if ((FULL_S || u < CT * VT) && g_in != nullptr) {
      const int Ct = u % CT, Vt = u / CT;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        accS[i][e] = g_in[(size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r];
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
  const E* iQL = reinterpret_cast<const E*>(img + IMG::QL);
  const E* iKT = reinterpret_cast<const E*>(img + IMG::KT);
  const E* iP = reinterpret_cast<const E*>(img + IMG::P);
  const float* iLC = reinterpret_cast<const float*>(img + IMG::LC);

  if (n_hi > n_lo) {
    issue_copy(n_hi - 1);
    load_do(n_hi - 1);
  }
  for (int n = n_hi - 1; n >= n_lo; --n) {
    __builtin_amdgcn_s_waitcnt(0);  // image and dO of chunk n
    stage_do(n);
    lds_barrier();
    // the gradient of this chunk's end state, for the per-chunk products: dS' [c][v]
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (!MAPW && (FULL_S || u < CT * VT)) {
        const int Ct = u % CT, Vt = u / CT;
        E* ck = static_cast<E*>(p.ckdS) + (rec0 + n * rstride) * D * D + vb0 + 16 * Vt + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) ck[(size_t)(16 * Ct + 4 * g4 + e) * D] = from_f32<E>(accS[i][e]);
      }
    }
    // ---- fragments of this chunk
    RowFrag<E, C> fpt;   // P^T row t_row
    RowFrag<E, D> fkt;   // Ktil row t_row
    RowFrag<E, C> fqlt[NCTW], fwt[NCTW];
    f32x4 flc[NCTW];
    if (has_u) {
      load_frag_t<C, C>(fpt, iP, 16 * R, r, g4);
      fpt.mask_below(t_row, g4);  // P[j][t] vanishes for j < t
      load_frag_t<D, C>(fkt, iKT, 16 * R, r, g4);
    }
#pragma unroll
    for (int jj = 0; jj < NCTW; ++jj) {
      const int Ct = (wave % CTW) + CTW * jj;
      load_frag_t<C, D>(fqlt[jj], iQL, 16 * Ct, r, g4);
      load_frag_t<C, D>(fwt[jj], iW, 16 * Ct, r, g4);
      flc[jj] = *reinterpret_cast<const f32x4*>(iLC + 16 * Ct + 4 * g4);
    }
    lds_barrier();  // every wave holds its fragments: the image may be overwritten
    if (n > n_lo) {
      issue_copy(n - 1);
      load_do(n - 1);
    }
    const E* sdo = sDO[n & 1];
    // ---- dU = P^T dO + Ktil dS'
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (FULL_U || u < RT * VT) {
        const int Vt = u / RT;
        RowFrag<E, C> fo;
        fo.load(sdo + (16 * Vt + r) * LU, g4);
        RowFrag<E, D> fs;
        fs.load(sS + (16 * Vt + r) * LS, g4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mma<C>(acc, fpt, fo);
        mma<D>(acc, fkt, fs);
        store4(&sDU[(16 * Vt + r) * LU + 16 * R + 4 * g4], acc[0], acc[1], acc[2], acc[3]);
        if constexpr (!MAPW) {
          E* du = static_cast<E*>(p.dU) + (rec0 + n * rstride) * C * D + vb0 + 16 * Vt + r;  // dU [t][v]
#pragma unroll
          for (int e = 0; e < 4; ++e) du[(size_t)(16 * R + 4 * g4 + e) * D] = from_f32<E>(acc[e]);
        }
      }
    }
    lds_barrier();  // sDU complete; every read of sS for this chunk is done
    // ---- dS = Diag(LC) dS' + QL^T dO - W^T dU
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (FULL_S || u < CT * VT) {
        const int Vt = u / CT;
        const int jj = i % NCTW;
        RowFrag<E, C> fo, fu;
        fo.load(sdo + (16 * Vt + r) * LU, g4);
        fu.load(sDU + (16 * Vt + r) * LU, g4);
        f32x4 neg = {0.f, 0.f, 0.f, 0.f};
        mma<C>(neg, fwt[jj], fu);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] = accS[i][e] * flc[jj][e] - neg[e];
        mma<C>(accS[i], fqlt[jj], fo);
      }
    }
    stage_state();
  }
  // the gradient of the start state: dS0, or a segment's reverse map
  float* g_out = seg == 0 && p.dS0 != nullptr ? p.dS0 + sbase : nullptr;
  if constexpr (MAPW)
    g_out = p.maps + ((size_t)bh * (p.nseg - 1) + (seg - 1)) * 3 * D * D;
  if (g_out != nullptr) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (FULL_S || u < CT * VT) {
        const int Ct = u % CT, Vt = u / CT;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          g_out[(size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r] = accS[i][e];
      }
    }
  }
}

// sum over a lane's elements of two fragments of the same rows
template <int K>
__device__ __forceinline__ float frag_dot(const RowFrag<__bf16, K>& a, const RowFrag<__bf16, K>& b) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < RowFrag<__bf16, K>::N; ++i)
#pragma unroll
    for (int e = 0; e < RowFrag<__bf16, K>::PER; ++e) acc = fmaf((float)a.v[i][e], (float)b.v[i][e], acc);
  return acc;
}
template <int K>
__device__ __forceinline__ float frag_dot(const RowFrag<float, K>& a, const RowFrag<float, K>& b) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < RowFrag<float, K>::N; ++i) acc = fmaf(a.v[i], b.v[i], acc);
  return acc;
}

// ------------------------------------------------------- per-chunk state products
// One 256-thread workgroup per chunk record.  In the NT products
// C[i][j] = sum_k A[i][k] B[j][k] (operands k-contiguous, element type, float
// accumulation), fragments loaded straight from the checkpoints, dO, dU and the
// record; U, as the forward walk rounded it, is checkpointed and staged in LDS:
//   dQL  = dO S^T:     A = dO rows t,           B = S rows c
//   dW   = -dU S^T:    A = dU rows t,           B = S rows c
//   dKt  = U dS'^T:    A = U rows t,            B = dS' rows c
//   dP   = dO U^T:     A = dO rows i,           B = U rows j      (j <= i)
//   dLC  = rowsum(dS' * S), from the S and dS' fragments of the dQL, dKt tiles
template <int D, int C, typename IO, typename E>
__global__ __launch_bounds__(256) void kda_bwd_prod_kernel(BwdProdParams p) {
  constexpr int PE = 16 / (int)sizeof(E);
  constexpr int LD = D + PE;
  constexpr int CT = D / 16, RT = C / 16;
  __shared__ __attribute__((aligned(16))) E sU[C * LD];  // U rows t, k = v
  // column tiles of S and dS' (16 rows each), two buffers (used when C = 64)
  constexpr int STG = C == 64 ? 16 * D : 1;
  __shared__ __attribute__((aligned(16))) E sSt0[STG];
  __shared__ __attribute__((aligned(16))) E sDt0[STG];
  __shared__ __attribute__((aligned(16))) E sSt1[STG];
  __shared__ __attribute__((aligned(16))) E sDt1[STG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int rec = blockIdx.x;
  const RecTok rt = rec_tokens(rec, p.B, p.T, p.H, C, p.seqs);
  if (rt.nval == 0) return;  // an unused slot: nothing reads its products
  const int h = rt.h;
  const size_t HD = (size_t)p.H * D;
  const E* ckS = static_cast<const E*>(p.ckS) + (size_t)rec * ((size_t)D * D + (size_t)C * D);  // [c][v]
  const E* ckU = ckS + (size_t)D * D;                                                         // [t][v]
  const E* ckdS = static_cast<const E*>(p.ckdS) + (size_t)rec * D * D;     // [c][v]
  const E* gdU = static_cast<const E*>(p.dU) + (size_t)rec * C * D;         // [t][v]
  const IO* gdO = static_cast<const IO*>(p.dO) + (size_t)rt.tok * HD + (size_t)h * D;
  const int nval = rt.nval;

  // dO fragment of row t (zero past the end of the sequence)
  auto load_do = [&](RowFrag<E, D>& f, int t) {
    if (t < nval) {
      if constexpr (sizeof(IO) == sizeof(E)) {
        f.load(reinterpret_cast<const E*>(gdO + (size_t)t * HD), g4);
      }
    } else {
      f = RowFrag<E, D>{};
    }
  };

  // Wave w owns t-tile Rt = w % RT (its row strips of dO, dU and U are
  // loaded once) and every WPR-th column tile from w / RT, so the four waves
  // read each checkpoint strip at about the same time (once from memory).
  constexpr int WPR = 4 / RT;  // waves per t-tile
  const int Rt = wave % RT, sub = wave / RT;
  // ---- U (as the forward walk rounded it) into LDS, 16-byte pieces
  for (int it = tid; it < C * D / PE; it += 256) {
    const int t = it / (D / PE), c0 = PE * (it % (D / PE));
    *reinterpret_cast<u32x4*>(&sU[t * LD + c0]) = *reinterpret_cast<const u32x4*>(ckU + (size_t)t * D + c0);
  }
  __syncthreads();

  // ---- dQL, dW, dKt: tiles (t, c); dP: tiles (i, j) with j <= i
  E* dQL = static_cast<E*>(p.dQL) + (size_t)rec * C * D;
  E* dW = static_cast<E*>(p.dW) + (size_t)rec * C * D;
  E* dKt = static_cast<E*>(p.dKt) + (size_t)rec * C * D;
  E* dP = static_cast<E*>(p.dP) + (size_t)rec * C * C;
  RowFrag<E, D> fdo, fdu, fu;
  load_do(fdo, 16 * Rt + r);
  fdu.load(gdU + (size_t)(16 * Rt + r) * D, g4);
  fu.load(sU + (16 * Rt + r) * LD, g4);
  // the products of column tile Ct, from this lane's fragments fs, fds of rows
  // 16 Ct + r of S and dS'
  auto col_tile = [&](int Ct, const RowFrag<E, D>& fs, const RowFrag<E, D>& fds) {
    // tiles formed transposed, (c, t): lane (r, g4) holds columns 16 Ct + 4 g4 + e
    // of row t = 16 Rt + r, stored as 4 contiguous elements
    f32x4 aq = {0.f, 0.f, 0.f, 0.f}, aw = aq, ak = aq;
    mma<D>(aq, fs, fdo);
    mma<D>(aw, fs, fdu);
    mma<D>(ak, fds, fu);
    const size_t o = (size_t)(16 * Rt + r) * D + 16 * Ct + 4 * g4;
    store4(dQL + o, aq[0], aq[1], aq[2], aq[3]);
    store4(dW + o, -aw[0], -aw[1], -aw[2], -aw[3]);
    store4(dKt + o, ak[0], ak[1], ak[2], ak[3]);
    if (Rt == 0) {
      // dLC of rows c = 16 Ct + r: this lane's pieces of the row are the same
      // elements of fs and fds, the rest sit in the lanes of the other g4
      const float sum = frag_dot(fs, fds);
      float tot = sum + __shfl_xor(sum, 16, 64);
      tot += __shfl_xor(tot, 32, 64);
      if (g4 == 0) p.dLC[(size_t)rec * D + 16 * Ct + r] = tot;
    }
  };
  if constexpr (WPR == 1) {
    // Every wave sweeps every column tile at the same time: the 16 rows of S and dS'
    // of tile Ct are copied once into LDS (asynchronous global-to-LDS loads, one
    // 16-byte piece per thread and matrix, swizzled so the fragment reads spread
    // over the banks), the copy of tile Ct + 1 running while tile Ct computes.
    using SW = Swz<E, D>;
    constexpr int NCH = 16 * D * (int)sizeof(E) / 16;  // pieces per matrix tile
    static_assert(NCH <= 256, "one piece per thread and matrix");
    auto stage = [&](int Ct, E* dstS, E* dstD) {
      if (tid < NCH) {
        constexpr int RC = SW::RC;
        const int row = tid / RC, pos = tid % RC;
        const size_t src = (size_t)(16 * Ct + row) * D + (size_t)((pos ^ (row & (RC - 1))) * SW::EPC);
        __builtin_amdgcn_global_load_lds((const glb_void_t*)(ckS + src), (lds_void_t*)(dstS + 64 * wave * SW::EPC),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const glb_void_t*)(ckdS + src), (lds_void_t*)(dstD + 64 * wave * SW::EPC),
                                         16, 0, 0);
      }
    };
    // two buffers at fixed offsets (the compiler keeps the copies in flight apart
    // from the reads of the other buffer)
    auto tile = [&](int Ct, E* curS, E* curD, E* nxtS, E* nxtD) {
      __builtin_amdgcn_s_waitcnt(0);  // this thread's pieces of tile Ct (and older stores)
      __syncthreads();                // tile Ct is in LDS; every read of the other buffer is done
      if (Ct + 1 < CT) stage(Ct + 1, nxtS, nxtD);
      RowFrag<E, D> fs, fds;
      load_swz<D>(fs, curS, r, g4);
      load_swz<D>(fds, curD, r, g4);
      col_tile(Ct, fs, fds);
    };
    stage(0, sSt0, sDt0);
    for (int Ct = 0; Ct < CT; Ct += 2) {
      tile(Ct, sSt0, sDt0, sSt1, sDt1);
      if (Ct + 1 < CT) tile(Ct + 1, sSt1, sDt1, sSt0, sDt0);
    }
  } else {
    for (int Ct = sub; Ct < CT; Ct += WPR) {
      RowFrag<E, D> fs, fds;
      fs.load(ckS + (size_t)(16 * Ct + r) * D, g4);
      fds.load(ckdS + (size_t)(16 * Ct + r) * D, g4);
      col_tile(Ct, fs, fds);
    }
  }
  for (int Jt = sub; Jt < RT; Jt += WPR) {
    const int It = Rt;
    // transposed tile (j, i): lane (r, g4) holds columns j = 16 Jt + 4 g4 + e of
    // row i = 16 It + r
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (Jt <= It) {
      RowFrag<E, D> fb;
      fb.load(sU + (16 * Jt + r) * LD, g4);
      mma<D>(acc, fb, fdo);
    }
    const int i = 16 * It + r, j0 = 16 * Jt + 4 * g4;
    store4(dP + (size_t)i * C + j0, j0 <= i ? acc[0] : 0.f, j0 + 1 <= i ? acc[1] : 0.f,
           j0 + 2 <= i ? acc[2] : 0.f, j0 + 3 <= i ? acc[3] : 0.f);
  }
}

// ------------------------------------------------------------ T-side products
// Persistent: each 512-thread workgroup (two waves per SIMD, so one's LDS reads
// and barriers overlap the other's products) takes records blockIdx.x,
// blockIdx.x + gridDim.x, ...; the global loads of its next record go into
// registers while the current one computes from LDS.  float32 matrix-core
// products (16x16x4, one element per lane and step, so operands read along either
// index):
//   dT = dW Bk^T + dU Bv^T   (j <= i),   Y = dT T^T,   dA = -T^T Y   (j < i)
//   dBk = T^T dW,   dBv = T^T dU
// Bk = beta K Lambda and Bv = beta V are rebuilt from the front end's outputs.
template <int D, int C, typename E>
__global__ __launch_bounds__(512) void kda_bwd_t_kernel(BwdTParams p) {
  constexpr int NT = 512, NW = NT / 64;
  constexpr int LD = D + 4;                  // float rows of D
  constexpr int LC = C + 4;                  // float rows of C
  constexpr int LB = D + 16 / (int)sizeof(E);  // E rows of D
  constexpr int CT = D / 16, RT = C / 16;
  constexpr int BKY = (C * LB * (int)sizeof(E) > C * LC * 4) ? C * LB * (int)sizeof(E) : C * LC * 4;
  // per-thread shares of one record's inputs
  constexpr int N4 = (C * D / 4 + NT - 1) / NT;  // dW in float4 pieces
  constexpr int N8 = (C * D / 8 + NT - 1) / NT;  // dU, k, v, Gamma in 8-element pieces
  constexpr int NC = (C * C / 4 + NT - 1) / NT;  // T^T in float4 pieces
  __shared__ __attribute__((aligned(16))) float sdW[C * LD];
  __shared__ __attribute__((aligned(16))) E sdU[C * LB];  // dU in its stored element type
  __shared__ __attribute__((aligned(16))) float sTt[C * LC];
  __shared__ __attribute__((aligned(16))) float sdT[C * LC];
  __shared__ __attribute__((aligned(16))) char sBkY[BKY];  // Bk [C][LB] E, later Y [C][LC] float
  __shared__ __attribute__((aligned(16))) E sBv[C * LB];
  E* sBk = reinterpret_cast<E*>(sBkY);

  const size_t HD = (size_t)p.H * D;
  const size_t plane = (size_t)p.B * p.T * HD;
  const int nrec = p.B * p.H * p.NT;

  struct Stage {
    f32x4 dw[N4];
    float du[N8][8], kk[N8][8], vv[N8][8], gg[N8][8];
    float bt[N8];
    f32x4 tt[NC];
  };
  auto load_stage = [&](int rec, int tid, Stage& S) {
    // (an unused slot of a packed batch reads token row 0 with beta = 0; nothing
    // reads what it produces)
    const RecTok rt = rec_tokens(rec, p.B, p.T, p.H, C, p.seqs);
    const int h = rt.h;
    const float* gdW = static_cast<const float*>(p.dW) + (size_t)rec * C * D;
    const E* gdU = static_cast<const E*>(p.dU) + (size_t)rec * C * D;  // [t][v]
    const float* gTt = static_cast<const float*>(p.tT) + (size_t)rec * C * C;
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const int it = tid + NT * i;
      if (it < C * D / 4) S.dw[i] = *reinterpret_cast<const f32x4*>(gdW + 4 * (size_t)it);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int it = tid + NT * i;
      if (it < C * C / 4) S.tt[i] = *reinterpret_cast<const f32x4*>(gTt + 4 * (size_t)it);
    }
#pragma unroll
    for (int i = 0; i < N8; ++i) {
      const int it = tid + NT * i;
      if (it < C * D / 8) {
        const int t = it / (D / 8), c8 = 8 * (it % (D / 8));
        load8(gdU + (size_t)t * D + c8, S.du[i]);
        // rows past the end of the sequence read the last row and take beta = 0
        // (no branch around the loads, so they stay in flight)
        const int tc = t < rt.nval ? t : (rt.nval > 0 ? rt.nval - 1 : 0);
        const size_t row = ((size_t)rt.tok + tc) * HD + (size_t)h * D + c8;
        load8(static_cast<const E*>(p.y) + plane + row, S.kk[i]);
        load8(static_cast<const E*>(p.y) + 2 * plane + row, S.vv[i]);
        load8(p.gam + row, S.gg[i]);
        const float bv = p.beta[((size_t)rt.tok + tc) * p.H + h];
        S.bt[i] = t < rt.nval ? bv : 0.f;
      }
    }
  };
  // into LDS; Bk = beta k exp(Gamma), Bv = beta v (zero past the end of the sequence)
  auto store_stage = [&](int tid, const Stage& S) {
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const int it = tid + NT * i;
      if (it < C * D / 4) {
        const int t = it / (D / 4), c4 = 4 * (it % (D / 4));
        *reinterpret_cast<f32x4*>(&sdW[t * LD + c4]) = S.dw[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int it = tid + NT * i;
      if (it < C * C / 4) {
        const int j = it / (C / 4), i4 = 4 * (it % (C / 4));
        *reinterpret_cast<f32x4*>(&sTt[j * LC + i4]) = S.tt[i];
      }
    }
#pragma unroll
    for (int i = 0; i < N8; ++i) {
      const int it = tid + NT * i;
      if (it < C * D / 8) {
        const int t = it / (D / 8), c8 = 8 * (it % (D / 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sdU[t * LB + c8 + e] = from_f32<E>(S.du[i][e]);
          sBk[t * LB + c8 + e] = from_f32<E>(S.bt[i] * S.kk[i][e] * __builtin_amdgcn_exp2f(S.gg[i][e]));
          sBv[t * LB + c8 + e] = from_f32<E>(S.bt[i] * S.vv[i][e]);
        }
      }
    }
  };

  int rec = blockIdx.x;
  Stage S;
  if (rec < nrec) load_stage(rec, threadIdx.x, S);
  while (rec < nrec) {
    // the thread's indices, opaque per record so that their address arithmetic
    // stays inside the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g4 = lane >> 4;
    store_stage(tid, S);
    __syncthreads();
    const int next = rec + (int)gridDim.x;
    if (next < nrec) load_stage(next, tid, S);

    // ---- dT (i, j) for j <= i
    for (int tile = wave; tile < RT * RT; tile += NW) {
      const int It = tile / RT, Jt = tile % RT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc;
      if (Jt <= It) {
        for (int k = 0; k < D; k += 4) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sdW[(16 * It + r) * LD + k + g4],
                                                     to_f32(sBk[(16 * Jt + r) * LB + k + g4]), acc, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(to_f32(sdU[(16 * It + r) * LB + k + g4]),
                                                      to_f32(sBv[(16 * Jt + r) * LB + k + g4]), acc2, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += acc2[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * It + 4 * g4 + e, j = 16 * Jt + r;
        sdT[i * LC + j] = j <= i ? acc[e] : 0.f;
      }
    }
    __syncthreads();  // dT complete; Bk, Bv dead
    float* sY = reinterpret_cast<float*>(sBkY);
    // ---- Y = dT T^T:  Y[i][j] = sum_m dT[i][m] T^T[m][j]
    for (int tile = wave; tile < RT * RT; tile += NW) {
      const int It = tile / RT, Jt = tile % RT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < C; k += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sdT[(16 * It + r) * LC + k + g4],
                                                   sTt[(k + g4) * LC + 16 * Jt + r], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sY[(16 * It + 4 * g4 + e) * LC + 16 * Jt + r] = acc[e];
    }
    __syncthreads();
    // ---- dA = -T^T Y  (j < i)
    float* gdA = static_cast<float*>(p.dA) + (size_t)rec * C * C;
    for (int tile = wave; tile < RT * RT; tile += NW) {
      const int It = tile / RT, Jt = tile % RT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (Jt <= It)
        for (int k = 0; k < C; k += 4)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sTt[(16 * It + r) * LC + k + g4],
                                                     sY[(k + g4) * LC + 16 * Jt + r], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * It + 4 * g4 + e, j = 16 * Jt + r;
        gdA[(size_t)i * C + j] = j < i ? -acc[e] : 0.f;
      }
    }
    // ---- dBk = T^T dW,  dBv = T^T dU  (tiles (j, c))
    float* gdBk = static_cast<float*>(p.dBk) + (size_t)rec * C * D;
    float* gdBv = static_cast<float*>(p.dBv) + (size_t)rec * C * D;
    for (int tile = wave; tile < RT * CT; tile += NW) {
      const int Jt = tile / CT, Ct = tile % CT;
      f32x4 ak = {0.f, 0.f, 0.f, 0.f}, av = ak;
      for (int k = 0; k < C; k += 4) {
        const float a = sTt[(16 * Jt + r) * LC + k + g4];
        ak = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sdW[(k + g4) * LD + 16 * Ct + r], ak, 0, 0, 0);
        av = __builtin_amdgcn_mfma_f32_16x16x4f32(a, to_f32(sdU[(k + g4) * LB + 16 * Ct + r]), av, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const size_t o = (size_t)(16 * Jt + 4 * g4 + e) * D + 16 * Ct + r;
        gdBk[o] = ak[e];
        gdBv[o] = av[e];
      }
    }
    __syncthreads();  // LDS is reused by the next record
    rec = next;
  }
}

// bf16 records: the same products as element-type matrix-core products
// (16x16x32, operands k-contiguous from swizzled LDS images, float accumulation),
// the float32 inputs rounded to bf16 as the forward rounds T and its operands.
// One 512-thread workgroup per chunk record.  LDS images (rows, k): W [i][c] of
// dW, U [i][c] of dU, Bk [j][c], Bv [j][c], T^T [i][m], dT^T [l][m], Y [m][j]; the
// rows of a transposed operand (T, dT, Y^T, W^T, U^T) are read down the columns of
// the stored image with the transposing read.  The products, in the NT form
// C[a][b] = sum_k A[a][k] B[b][k]:
//   dT  = dW Bk^T + dU Bv^T   A = W, U rows i;     B = Bk, Bv rows j      (j <= i)
//   Y^T = T dT^T              A = T rows j;        B = dT rows m
//   dA  = -T^T Y              A = T^T rows i;      B = Y^T rows j         (j < i)
//   dBk = T^T dW,  dBv = T^T dU   A = T^T rows j;  B = W^T, U^T rows c
template <int D, int C>
__global__ __launch_bounds__(512) void kda_bwd_t16_kernel(BwdTParams p) {
  constexpr int NT = 512, NW = NT / 64;
  constexpr int CT = D / 16, RT = C / 16;
  using SD = Swz<__bf16, D>;
  using SC = Swz<__bf16, C>;
  // One region holds the images of dW, dU, Bk, Bv for the dT products; Y then
  // takes the place of Bk (dW and dU stay for the dBk, dBv products, which read
  // them as transposed fragments); T^T and dT sit beside it.  T itself is read as
  // transposed fragments of T^T.  80 KB at C = 64, D = 128, so two workgroups
  // share a compute unit.
  constexpr int REG = 2 * C * D + (C * C > 2 * C * D ? C * C : 2 * C * D);
  __shared__ __attribute__((aligned(16))) __bf16 reg[REG];
  __shared__ __attribute__((aligned(16))) __bf16 iTt[C * C];
  __shared__ __attribute__((aligned(16))) __bf16 idTt[C * C];  // dT^T
  __bf16* iW = reg;
  __bf16* iU = reg + C * D;
  __bf16* iBk = reg + 2 * C * D;
  __bf16* iBv = reg + 3 * C * D;
  __bf16* iY = iBk;  // Y, after the dT products

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int rec = blockIdx.x;
  const RecTok rt = rec_tokens(rec, p.B, p.T, p.H, C, p.seqs);
  if (rt.nval == 0) return;  // an unused slot: nothing reads its products
  const int h = rt.h;
  const size_t HD = (size_t)p.H * D;
  const size_t plane = (size_t)p.B * p.T * HD;

  // ---- images
  const __bf16* gdW = static_cast<const __bf16*>(p.dW) + (size_t)rec * C * D;
  const __bf16* gdU = static_cast<const __bf16*>(p.dU) + (size_t)rec * C * D;  // [t][v]
  const __bf16* gTt = static_cast<const __bf16*>(p.tT) + (size_t)rec * C * C;  // [j][i] = T[i][j]
  for (int it = tid; it < C * D / 4; it += NT) {
    const int t = it / (D / 4), c4 = 4 * (it % (D / 4));
    // 4 elements inside one 16-byte chunk of the image row
    *reinterpret_cast<bf16x4*>(&iW[SD::at(t, c4)]) =
        *reinterpret_cast<const bf16x4*>(gdW + (size_t)t * D + c4);
  }
  for (int it = tid; it < C * D / 8; it += NT) {
    const int t = it / (D / 8), c8 = 8 * (it % (D / 8));
    const bf16x8 u = *reinterpret_cast<const bf16x8*>(gdU + (size_t)t * D + c8);
    *reinterpret_cast<bf16x8*>(&iU[SD::at(t, c8)]) = u;  // 8 elements = one 16-byte chunk
  }
  for (int it = tid; it < C * C / 4; it += NT) {
    const int a = it / (C / 4), b4 = 4 * (it % (C / 4));
    // T^T[a][b4 .. b4 + 3], inside one 16-byte chunk of the image row
    *reinterpret_cast<bf16x4*>(&iTt[SC::at(a, b4)]) =
        *reinterpret_cast<const bf16x4*>(gTt + (size_t)a * C + b4);
  }
  // Bk = beta k exp(Gamma), Bv = beta v; rows past the end of the sequence read
  // the last row and take beta = 0
  for (int it = tid; it < C * D / 8; it += NT) {
    const int t = it / (D / 8), c8 = 8 * (it % (D / 8));
    const int tc = t < rt.nval ? t : rt.nval - 1;
    const size_t row = ((size_t)rt.tok + tc) * HD + (size_t)h * D + c8;
    float kk[8], vv[8], gg[8];
    load8(static_cast<const __bf16*>(p.y) + plane + row, kk);
    load8(static_cast<const __bf16*>(p.y) + 2 * plane + row, vv);
    load8(p.gam + row, gg);
    const float bv = p.beta[((size_t)rt.tok + tc) * p.H + h];
    const float bt = t < rt.nval ? bv : 0.f;
    bf16x8 xk, xv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xk[e] = (__bf16)(bt * kk[e] * __builtin_amdgcn_exp2f(gg[e]));
      xv[e] = (__bf16)(bt * vv[e]);
    }
    *reinterpret_cast<bf16x8*>(&iBk[SD::at(t, c8)]) = xk;
    *reinterpret_cast<bf16x8*>(&iBv[SD::at(t, c8)]) = xv;
  }
  __syncthreads();

  // ---- dT (i, j), zero above the diagonal
  for (int tile = wave; tile < RT * RT; tile += NW) {
    const int It = tile / RT, Jt = tile % RT;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (Jt <= It) {
      RowFrag<__bf16, D> fa, fb;
      load_swz<D>(fa, iW, 16 * It + r, g4);
      load_swz<D>(fb, iBk, 16 * Jt + r, g4);
      mma<D>(acc, fa, fb);
      load_swz<D>(fa, iU, 16 * It + r, g4);
      load_swz<D>(fb, iBv, 16 * Jt + r, g4);
      mma<D>(acc, fa, fb);
    }
    // rows i .. i + 3 of column j: 4 consecutive elements of row j of dT^T
    const int i0 = 16 * It + 4 * g4, j = 16 * Jt + r;
    bf16x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (__bf16)(j <= i0 + e ? acc[e] : 0.f);
    *reinterpret_cast<bf16x4*>(&idTt[SC::at(j, i0)]) = x;
  }
  __syncthreads();  // the images of Bk and Bv are dead
  // ---- Y^T (j, m) = sum_l T[j][l] dT[m][l], T rows read down the columns of T^T
  for (int tile = wave; tile < RT * RT; tile += NW) {
    const int Jt = tile / RT, Mt = tile % RT;
    RowFrag<__bf16, C> fa, fb;
    load_frag_t<C, C>(fa, iTt, 16 * Jt, r, g4);
    load_swz_tr<C, C>(fb, idTt, 16 * Mt, r, g4);  // dT rows: columns of dT^T
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mma<C>(acc, fa, fb);
    // Y^T rows j .. j + 3 of column m: 4 consecutive elements of row m of Y
    bf16x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (__bf16)acc[e];
    *reinterpret_cast<bf16x4*>(&iY[SC::at(16 * Mt + r, 16 * Jt + 4 * g4)]) = x;
  }
  __syncthreads();
  // ---- dA (i, j) = -sum_m T^T[i][m] Y^T[j][m]  (j < i)
  __bf16* gdA = static_cast<__bf16*>(p.dA) + (size_t)rec * C * C;
  for (int tile = wave; tile < RT * RT; tile += NW) {
    const int It = tile / RT, Jt = tile % RT;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (Jt <= It) {
      RowFrag<__bf16, C> fa, fb;
      load_swz<C>(fa, iTt, 16 * It + r, g4);
      load_swz_tr<C, C>(fb, iY, 16 * Jt, r, g4);  // Y^T rows: columns of Y
      mma<C>(acc, fa, fb);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * It + 4 * g4 + e, j = 16 * Jt + r;
      gdA[(size_t)i * C + j] = (__bf16)(j < i ? -acc[e] : 0.f);
    }
  }
  // ---- dBk (j, c) = sum_i T^T[j][i] dW^T[c][i],  dBv likewise with dU (dW^T and
  // dU^T rows read as transposed fragments of the dW, dU images)
  __bf16* gdBk = static_cast<__bf16*>(p.dBk) + (size_t)rec * C * D;
  __bf16* gdBv = static_cast<__bf16*>(p.dBv) + (size_t)rec * C * D;
  for (int tile = wave; tile < RT * CT; tile += NW) {
    const int Jt = tile / CT, Ct = tile % CT;
    RowFrag<__bf16, C> ft, fw, fu;
    load_swz<C>(ft, iTt, 16 * Jt + r, g4);
    load_swz_tr<C, D>(fw, iW, 16 * Ct, r, g4);
    load_swz_tr<C, D>(fu, iU, 16 * Ct, r, g4);
    f32x4 ak = {0.f, 0.f, 0.f, 0.f}, av = ak;
    mma<C>(ak, ft, fw);
    mma<C>(av, ft, fu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t o = (size_t)(16 * Jt + 4 * g4 + e) * D + 16 * Ct + r;
      gdBk[o] = (__bf16)ak[e];
      gdBv[o] = (__bf16)av[e];
    }
  }
}

// ------------------------------------------ pair and element terms, factored
// The pair terms of A and P,
//   rK_i = sum_{j<i} dA_ij k_j E_ij,   rQ_i = sum_{j<=i} dP_ij k_j E_ij,
//   cK_j = sum_{i>=j} E_ij (beta_i dA_ij k_i + dP_ij q'_i)          (per channel),
// with E_ij = exp(Gamma_i - Gamma_j) factored as in the forward preparation:
// for i in 16-token block p and j in block q, with m_p the middle of block p's
// log-decay range,  E_ij = a_i F_pq b_j,  a_i = exp(Gamma_i - m_p),
// b_j = exp(m_q - Gamma_j),  F_pq = exp(m_p - m_q) (1 for p = q).  Then per block
// pair (p, q <= p) and channel tile, float32 matrix-core products:
//   rK_p += F_pq (dA_pq (K b)_q),   rQ_p += F_pq (dP_pq (K b)_q),
//   cK_q += F_pq (dA_pq^T (beta K a)_p + dP_pq^T (Q' a)_p),
// and rK, rQ take the factor a, cK the factor b.  dA and dP are exactly zero above
// their diagonals, so the pairs j > i (whose a_i b_j exceed 1) add nothing.  The
// pair factor F_pq = exp(m_p - m_q) (p > q) is exp(-(s_p + s_q)/2) or smaller and
// may underflow where the products it scales do not, so it is applied in two
// steps, exp(-s/2) of the block whose operand carries exp(+s/2) first (with G_q
// the cumulative decay before block q):
//   rK_p, rQ_p:  (. exp(-s_q/2)) exp(m_p - G_{q+1}),   cK_q:  (. exp(-s_p/2)) exp(G_p - m_q),
// both factors <= 1.  a and b lie within 2^(+-s/2) for a block span s (log2
// units), so every operand and partial sum of the products is bounded by
//   C max(|dA| |k|, |dP| |k|, |beta| |dA| |k| + |dP| |q'|) 2^(s/2)
// with each maximum taken over the chunk.  A chunk whose widest span or whose
// bound exceeds what float32 holds with room to spare (span 240, bound 2^120) is
// listed for the exact kernel; the bound comes from the chunk's own values, so
// wide spans with ordinary gradients stay factored.
// One workgroup per chunk record; wave w owns channels [16 w, 16 w + 16).  Lane
// (r, g4) holds the operands of rows 4 s + g4 (s < C / 4) of its channel 16 w + r
// (the matrix-core B layout), and its results for rows 16 p + 4 g4 + e.  Row
// block by row block: the products that finish rK, rQ and cK of the block, which
// go through LDS once, then its element terms as in the exact kernel with thread
// (row, 4 adjacent channels) of the block, so that every input and output of
// that phase moves as one vector access per tensor.
constexpr float kBwdSpan2 = 240.f;   // widest block span factored (log2 units)
constexpr float kBwdBound2 = 120.f;  // log2 of the largest partial sum allowed

template <int D, int C, typename E>
__global__ __launch_bounds__(4 * D, D / 32 > 1 ? D / 32 : 1) void kda_bwd_pair_mma_kernel(BwdPairParams p) {
  constexpr int NTH = 4 * D;
  constexpr int NB = C / 16;
  constexpr int NS = C / 4;     // rows per lane in the B layout
  constexpr int LA = C + 2;     // dA, dP rows (row reads of 16 lanes x 4 columns spread over the banks)
  constexpr int LD = D + 4;     // dGamma rows
  constexpr int LT = D + 4;     // rows of the block's product results
  constexpr int CPT = D / 4;    // threads per row in the element phase
  // dA, dP in the record element type (they arrive in it, so bf16 is exact)
  __shared__ __attribute__((aligned(16))) E sreg[2 * C * LA];
  __shared__ __attribute__((aligned(16))) float sG[C * LD];         // dGamma
  // rK, rQ, cK sums of one row block [3][16][LT] (finally the dKt Ktil column partials)
  __shared__ __attribute__((aligned(16))) float sT[3 * 16 * LT];
  __shared__ float smid[NB * D];  // block midpoints per channel
  __shared__ float sGC[D];
  __shared__ float sB[C];
  // per wave: the widest block span of its channels, the largest |k|, |q'|, |dA|,
  // |dP| it holds; and the largest |beta| of the chunk
  __shared__ float smax[5][D / 16];
  __shared__ float smaxb;
  constexpr int NSG = NTH / D;  // token segments of the dg running sum
  constexpr int SL = C / NSG;   // tokens per segment
  __shared__ float sseg[NSG * D];  // segment totals of dGamma
  E* sdA = sreg;
  E* sdP = sreg + C * LA;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int c = 16 * wave + r;  // this lane's channel
  const int rec = blockIdx.x;
  const RecTok rt = rec_tokens(rec, p.B, p.T, p.H, C, p.seqs);
  if (rt.nval == 0) return;  // an unused slot of a packed batch
  const int h = rt.h;
  const size_t HD = (size_t)p.H * D;
  const size_t plane = (size_t)p.B * p.T * HD;
  const int nval = rt.nval;  // tokens of the sequence in this chunk
  auto row_of = [&](int t) { return ((size_t)rt.tok + t) * HD + (size_t)h * D; };
  // Gamma of row t (past the end of the sequence g = 0: Gamma keeps its last value)
  auto gam_at = [&](int t) { return p.gam[row_of(t < nval ? t : nval - 1) + c]; };
  const E* y = static_cast<const E*>(p.y);

  // ---- B-layout operands of this lane: rows 4 s + g4
  float gB[NS], kB[NS], qB[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int t = 4 * s + g4;
    const bool in = t < nval;
    gB[s] = gam_at(t);
    kB[s] = in ? to_f32(y[plane + row_of(t) + c]) : 0.f;
    qB[s] = in ? to_f32(y[row_of(t) + c]) : 0.f;
  }
  if (tid < C) sB[tid] = tid < nval ? p.beta[((size_t)rt.tok + tid) * p.H + h] : 0.f;
  // block boundaries G_1 .. G_NB (Gamma at the last row of each block: lane
  // (r, 3), s = 4 p + 3) and the midpoints m_p = (G_p + G_p+1) / 2, G_0 = 0
  float mid[NB], gbd[NB + 1];  // midpoints, block boundaries G_0 = 0, G_1, ...
  float mx[5] = {0.f, 0.f, 0.f, 0.f, 0.f};  // span, |k|, |q'|, |dA|, |dP| seen by this lane
  {
    float gprev = 0.f;
    gbd[0] = 0.f;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const float gend = __shfl(gB[4 * q + 3], 48 + r, 64);
      mid[q] = 0.5f * (gprev + gend);
      gbd[q + 1] = gend;
      mx[0] = fmaxf(mx[0], gprev - gend);
      gprev = gend;
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    mx[1] = fmaxf(mx[1], fabsf(kB[s]));
    mx[2] = fmaxf(mx[2], fabsf(qB[s]));
  }
  // dA and dP into LDS
  const E* gdA = static_cast<const E*>(p.dA) + (size_t)rec * C * C;
  const E* gdP = static_cast<const E*>(p.dP) + (size_t)rec * C * C;
  for (int it = tid; it < C * C / 4; it += NTH) {
    const int i = it / (C / 4), j4 = 4 * (it % (C / 4));
    const f32x4 va = load4v(gdA + (size_t)i * C + j4);
    const f32x4 vp = load4v(gdP + (size_t)i * C + j4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sdA[i * LA + j4 + e] = from_f32<E>(va[e]);
      sdP[i * LA + j4 + e] = from_f32<E>(vp[e]);
      mx[3] = fmaxf(mx[3], fabsf(va[e]));
      mx[4] = fmaxf(mx[4], fabsf(vp[e]));
    }
  }
  if (g4 == 0) {
#pragma unroll
    for (int q = 0; q < NB; ++q) smid[q * D + c] = mid[q];
  }
#pragma unroll
  for (int m = 0; m < 5; ++m) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx[m] = fmaxf(mx[m], __shfl_xor(mx[m], o, 64));
    if (lane == 0) smax[m][wave] = mx[m];
  }
  if (wave == 0) {  // the beta loads above are lanes tid < C of wave 0
    float mb = tid < C ? fabsf(sB[tid]) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o, 64));
    if (lane == 0) smaxb = mb;
  }
  __syncthreads();
  bool anyfat;
  {
    float m[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < D / 16; ++w)
#pragma unroll
      for (int k = 0; k < 5; ++k) m[k] = fmaxf(m[k], smax[k][w]);
    const float span = m[0], mk = m[1], mq = m[2], ma = m[3], mp = m[4];
    const float bound = fmaxf(fmaxf(ma * mk, mp * mk), smaxb * ma * mk + mp * mq) * (float)C;
    // (an infinite or NaN bound fails the comparison and lists the chunk)
    anyfat = !(span <= kBwdSpan2 && bound <= __builtin_amdgcn_exp2f(kBwdBound2 - 0.5f * span));
  }
  if (anyfat) {
    if (tid == 0) {
      const unsigned slot = atomicAdd(p.ex_count, 1u);
      p.ex_list[slot] = (unsigned)rec;
    }
    return;
  }
  // K b, beta K a, Q' a
  float kb[NS], bka[NS], qa[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float m = mid[s / 4];
    const float a = __builtin_amdgcn_exp2f(gB[s] - m), bb = __builtin_amdgcn_exp2f(m - gB[s]);
    kb[s] = kB[s] * bb;
    bka[s] = sB[4 * s + g4] * kB[s] * a;
    qa[s] = qB[s] * a;
  }

  // ---- per row block pb: the block-pair products, then its element terms
  float* sdG = sG;  // [C][LD]
  const E* gdQL = static_cast<const E*>(p.dQL) + (size_t)rec * C * D;
  const E* gdKt = static_cast<const E*>(p.dKt) + (size_t)rec * C * D;
  const E* gdBk = static_cast<const E*>(p.dBk) + (size_t)rec * C * D;
  const E* gdBv = static_cast<const E*>(p.dBv) + (size_t)rec * C * D;
  // element phase: thread (row er of the block, channels c4 .. c4 + 3)
  const int er = tid / CPT, c4 = 4 * (tid % CPT);
  const size_t rowC = row_of(C - 1 < nval ? C - 1 : nval - 1);  // Gamma_C: the last row
  const f32x4 gC4 = load4v(p.gam + rowC + c4);
  f32x4 csum = {0.f, 0.f, 0.f, 0.f};  // sum over this thread's rows of dKt Ktil
#pragma unroll
  for (int pb = 0; pb < NB; ++pb) {
    f32x4 tK = {0.f, 0.f, 0.f, 0.f}, tQ = tK, tC = tK;
    // rK, rQ of rows in block pb: column blocks qb <= pb
#pragma unroll
    for (int qb = 0; qb <= pb; ++qb) {
      // F_pq = exp(-s_q/2) exp(m_p - G_{q+1}), applied one factor at a time
      const float F1 = pb == qb ? 1.f : __builtin_amdgcn_exp2f(gbd[qb + 1] - mid[qb]);
      const float F2 = pb == qb ? 1.f : __builtin_amdgcn_exp2f(mid[pb] - gbd[qb + 1]);
      f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = xk;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // rows (16 pb + r), columns (16 qb + 4 s + g4)
        const float a_ = to_f32(sdA[(16 * pb + r) * LA + 16 * qb + 4 * s + g4]);
        const float p_ = to_f32(sdP[(16 * pb + r) * LA + 16 * qb + 4 * s + g4]);
        xk = __builtin_amdgcn_mfma_f32_16x16x4f32(a_, kb[4 * qb + s], xk, 0, 0, 0);
        xq = __builtin_amdgcn_mfma_f32_16x16x4f32(p_, kb[4 * qb + s], xq, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tK[e] = fmaf(F2, xk[e] * F1, tK[e]);
        tQ[e] = fmaf(F2, xq[e] * F1, tQ[e]);
      }
    }
    // cK of columns in block pb: row blocks rb >= pb
#pragma unroll
    for (int rb = pb; rb < NB; ++rb) {
      // F_rp = exp(-s_r/2) exp(G_r - m_p), applied one factor at a time
      const float F1 = rb == pb ? 1.f : __builtin_amdgcn_exp2f(mid[rb] - gbd[rb]);
      const float F2 = rb == pb ? 1.f : __builtin_amdgcn_exp2f(gbd[rb] - mid[pb]);
      f32x4 xc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // transposed reads: rows (16 rb + 4 s + g4), columns (16 pb + r)
        const float at = to_f32(sdA[(16 * rb + 4 * s + g4) * LA + 16 * pb + r]);
        const float pt = to_f32(sdP[(16 * rb + 4 * s + g4) * LA + 16 * pb + r]);
        xc = __builtin_amdgcn_mfma_f32_16x16x4f32(at, bka[4 * rb + s], xc, 0, 0, 0);
        xc = __builtin_amdgcn_mfma_f32_16x16x4f32(pt, qa[4 * rb + s], xc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) tC[e] = fmaf(F2, xc[e] * F1, tC[e]);
    }
    // the element terms' inputs of row t = 16 pb + er, issued before the
    // block's sums go through LDS:
    // dQL, dKt, dBk, dBv, Gamma, q', k, v (rows past the end of the sequence read
    // the last row; q', k, v are zeroed there)
    const int t = 16 * pb + er;
    const bool in = t < nval;
    const size_t lo = (size_t)t * D + c4;
    const size_t o = row_of(in ? t : nval - 1) + c4;
    // (held in the element type until used: half the registers for bf16)
    using V4 = typename Vec4<E>::type;
    const V4 dql = *reinterpret_cast<const V4*>(gdQL + lo), dkt = *reinterpret_cast<const V4*>(gdKt + lo);
    const V4 dbk = *reinterpret_cast<const V4*>(gdBk + lo), dbv = *reinterpret_cast<const V4*>(gdBv + lo);
    const f32x4 gt = load4v(p.gam + o);
    const V4 qv = *reinterpret_cast<const V4*>(y + o), kv = *reinterpret_cast<const V4*>(y + plane + o),
             vv = *reinterpret_cast<const V4*>(y + 2 * plane + o);
    // the block's sums, rows 4 g4 + e of channel c, into LDS (the previous block's
    // element phase has read them: barrier at the end of each block)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sT[(0 * 16 + 4 * g4 + e) * LT + c] = tK[e];
      sT[(1 * 16 + 4 * g4 + e) * LT + c] = tQ[e];
      sT[(2 * 16 + 4 * g4 + e) * LT + c] = tC[e];
    }
    __syncthreads();
    // element terms of row t, channels c4 .. c4 + 3
    const f32x4 sK = *reinterpret_cast<const f32x4*>(&sT[(0 * 16 + er) * LT + c4]);
    const f32x4 sQ = *reinterpret_cast<const f32x4*>(&sT[(1 * 16 + er) * LT + c4]);
    const f32x4 sC = *reinterpret_cast<const f32x4*>(&sT[(2 * 16 + er) * LT + c4]);
    const f32x4 md = *reinterpret_cast<const f32x4*>(&smid[pb * D + c4]);
    const float bt = sB[t];
    float dg4[4], yq[4], yk[4], yv[4];
    float dbp = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float qq = in ? (float)qv[e] : 0.f, kk = in ? (float)kv[e] : 0.f, vx = in ? (float)vv[e] : 0.f;
      const float dqle = (float)dql[e], dkte = (float)dkt[e], dbke = (float)dbk[e], dbve = (float)dbv[e];
      const float a = __builtin_amdgcn_exp2f(gt[e] - md[e]), bb = __builtin_amdgcn_exp2f(md[e] - gt[e]);
      const float rK = a * sK[e], rQ = a * sQ[e], ckt = bb * sC[e];
      const float lam = __builtin_amdgcn_exp2f(gt[e]);
      const float ec = __builtin_amdgcn_exp2f(gC4[e] - gt[e]);
      const float ktil = kk * ec;
      csum[e] = fmaf(dkte, ktil, csum[e]);
      dg4[e] = dbke * bt * kk * lam + dqle * qq * lam - dkte * ktil + bt * kk * rK + qq * rQ - kk * ckt;
      yq[e] = lam * dqle + rQ;
      yk[e] = bt * lam * dbke + ec * dkte + bt * rK + ckt;
      yv[e] = bt * dbve;
      dbp += dbve * vx + dbke * kk * lam + kk * rK;
    }
    store4(&sdG[t * LD + c4], dg4[0], dg4[1], dg4[2], dg4[3]);
    if (in) {
      E* dy = static_cast<E*>(p.dy) + row_of(t) + c4;
      store4(dy, yq[0], yq[1], yq[2], yq[3]);
      store4(dy + plane, yk[0], yk[1], yk[2], yk[3]);
      store4(dy + 2 * plane, yv[0], yv[1], yv[2], yv[3]);
    }
    // dbeta of row t: the row's CPT threads are adjacent lanes of one wave
    dbp = group_sum<CPT>(dbp);
    if (c4 == 0 && in) p.dbeta_part[((size_t)rt.tok + t) * p.H + h] = dbp;
    __syncthreads();  // the block's sums are read
  }
  // dGamma_C: the dKt Ktil column sums over the chunk's rows, plus dLC LC
  store4(&sT[er * LT + c4], csum[0], csum[1], csum[2], csum[3]);
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) acc += sT[e2 * LT + tid];
    sGC[tid] = acc + p.dLC[(size_t)rec * D + tid] * __builtin_amdgcn_exp2f(p.gam[rowC + tid]);
  }
  __syncthreads();
  // dg: reverse running sum over the chunk.  Thread (channel cc, segment sg) takes
  // the SL tokens of segment sg: the segment totals go through LDS, then each
  // thread walks its segment backwards from the sum of the later segments.
  {
    const int cc = tid % D, sg = tid / D;
    float tot = 0.f;
#pragma unroll
    for (int t = SL * sg; t < SL * (sg + 1); ++t) tot += sdG[t * LD + cc];
    sseg[sg * D + cc] = tot;
    __syncthreads();
    float acc = sGC[cc];
    for (int s2 = NSG - 1; s2 > sg; --s2) acc += sseg[s2 * D + cc];
#pragma unroll
    for (int t = SL * (sg + 1) - 1; t >= SL * sg; --t) {
      acc += sdG[t * LD + cc];
      if (t < nval) p.dg[row_of(t) + cc] = acc;
    }
  }
}

// ------------------------------------------------- pair and element terms, dg
// Exact form, for the chunks the factored kernel above lists (decay spans too
// wide to factor): workgroup i takes listed record i, TPC = C / 16 threads per
// channel (adjacent lanes) and all D channels.  Per channel c, with E_ij = exp(Gamma_ic - Gamma_jc)
// for j <= i (at most 1, evaluated once per pair):
//   row i:    rK_i = sum_{j<i} dA_ij k_jc E_ij,   rQ_i = sum_{j<=i} dP_ij k_jc E_ij
//   column j: cK_j = sum_{i>=j} E_ij (beta_i dA_ij k_ic + dP_ij q'_ic)
// The C rows come in chunks of 4; thread t of a channel takes chunks t, 2 TPC - 1 - t,
// 2 TPC + t, 4 TPC - 1 - t (equal work), keeps its rows' sums and its share of
// every column sum in registers, and the column shares are added across the
// channel's lanes.  Then, per token t,
//   dq'  = Lambda dQL + rQ
//   dk   = beta Lambda dBk + exp(Gamma_C - Gamma) dKt + beta rK + cK
//   dv   = beta dBv
//   dGam = dBk Bk + dQL QL - dKt Ktil + beta k rK + q' rQ - k cK   (+ dGamma_C on the last row)
//   dbeta = sum_c (dBv v + dBk k Lambda + k rK)
// with dGamma_C = sum_t dKt Ktil + dLC LC, and dg = the reverse running sum of dGam.
template <int D, int C>
struct PairShape {
  static constexpr int TPC = C / 16;  // threads per channel (4 row chunks each)
  static constexpr int NTH = D * TPC;
};

template <int D, int C, typename E>
__global__ __launch_bounds__(D * (C / 16)) void kda_bwd_pair_kernel(BwdPairParams p) {
  constexpr int TPC = PairShape<D, C>::TPC;
  constexpr int NTH = PairShape<D, C>::NTH;
  constexpr int LA = C + 4;
  constexpr int LD = D + 4;
  constexpr int AP = 2 * C * LA > C * LD ? 2 * C * LA : C * LD;
  __shared__ __attribute__((aligned(16))) float sAP[AP];  // dA, dP; then cK, dbeta parts [C][LD]
  __shared__ __attribute__((aligned(16))) float sK[C * LD];
  __shared__ __attribute__((aligned(16))) float sQ[C * LD];  // later dGamma [C][LD]
  __shared__ __attribute__((aligned(16))) float sG[C * LD];
  __shared__ float sB[C];
  __shared__ float sGC[D];
  float* sdA = sAP;
  float* sdP = sAP + C * LA;

  const int tid = threadIdx.x;
  // workgroup i takes listed record i (the grid covers every record; most exit here)
  if (blockIdx.x >= *p.ex_count) return;
  const int rec = (int)p.ex_list[blockIdx.x];
  if (rec >= p.B * p.H * p.NT) return;  // (the list holds record indices only)
  const RecTok rt = rec_tokens(rec, p.B, p.T, p.H, C, p.seqs);
  if (rt.nval == 0) return;
  const int h = rt.h;
  const size_t HD = (size_t)p.H * D;
  const size_t plane = (size_t)p.B * p.T * HD;
  const int nval = rt.nval;  // tokens of the sequence in this chunk
  auto row_of = [&](int t) { return ((size_t)rt.tok + t) * HD + (size_t)h * D; };

  const E* gdA = static_cast<const E*>(p.dA) + (size_t)rec * C * C;
  const E* gdP = static_cast<const E*>(p.dP) + (size_t)rec * C * C;
  for (int it = tid; it < C * C / 4; it += NTH) {
    const int i = it / (C / 4), j4 = 4 * (it % (C / 4));
    *reinterpret_cast<f32x4*>(&sdA[i * LA + j4]) = load4v(gdA + (size_t)i * C + j4);
    *reinterpret_cast<f32x4*>(&sdP[i * LA + j4]) = load4v(gdP + (size_t)i * C + j4);
  }
  for (int it = tid; it < C * D / 4; it += NTH) {
    const int t = it / (D / 4), c4 = 4 * (it % (D / 4));
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qq = kk, gg = kk;
    if (t < nval) {
      const size_t o = row_of(t) + c4;
      const E* y = static_cast<const E*>(p.y);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qq[e] = to_f32(y[o + e]);
        kk[e] = to_f32(y[plane + o + e]);
      }
      gg = *reinterpret_cast<const f32x4*>(p.gam + o);
    } else if (nval > 0) {
      // past the end g = 0: Gamma keeps its last value
      gg = *reinterpret_cast<const f32x4*>(p.gam + row_of(nval - 1) + c4);
    }
    *reinterpret_cast<f32x4*>(&sK[t * LD + c4]) = kk;
    *reinterpret_cast<f32x4*>(&sQ[t * LD + c4]) = qq;
    *reinterpret_cast<f32x4*>(&sG[t * LD + c4]) = gg;
  }
  for (int t = tid; t < C; t += NTH)
    sB[t] = t < nval ? p.beta[((size_t)rt.tok + t) * p.H + h] : 0.f;
  __syncthreads();

  const int c = tid / TPC, tq = tid % TPC;
  // this thread's row chunks (4 rows each)
  int ck[4];
  ck[0] = tq;
  ck[1] = 2 * TPC - 1 - tq;
  ck[2] = 2 * TPC + tq;
  ck[3] = 4 * TPC - 1 - tq;
  float rK[4][4], rQ[4][4];
  float cacc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) cacc[j] = 0.f;
  for (int m = 0; m < 4; ++m) {
    const int i0 = 4 * ck[m];
    float gi[4], ki[4], qi[4], bi[4], ak[4], aq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      gi[r] = sG[(i0 + r) * LD + c];
      ki[r] = sK[(i0 + r) * LD + c];
      qi[r] = sQ[(i0 + r) * LD + c];
      bi[r] = sB[i0 + r];
      ak[r] = aq[r] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if (j < i0 + 4) {
        const float kj = sK[j * LD + c], gj = sG[j * LD + c];
        float col = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // pairs with j > i carry dA = dP = 0; the clamp keeps their E finite
          const float e = __builtin_amdgcn_exp2f(fminf(gi[r] - gj, 0.f));
          const float a = sdA[(i0 + r) * LA + j], pp = sdP[(i0 + r) * LA + j];
          const float ke = kj * e;
          ak[r] = fmaf(a, ke, ak[r]);
          aq[r] = fmaf(pp, ke, aq[r]);
          col = fmaf(e, fmaf(bi[r] * a, ki[r], pp * qi[r]), col);
        }
        cacc[j] += col;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rK[m][r] = ak[r];
      rQ[m][r] = aq[r];
    }
  }
  // column sums: add the shares of the channel's TPC lanes, then to LDS
#pragma unroll
  for (int j = 0; j < C; ++j) cacc[j] = group_sum<TPC>(cacc[j]);
  __syncthreads();  // every read of dA, dP is done
  float* sCK = sAP;  // [C][LD]
  if (tq == 0)
#pragma unroll
    for (int j = 0; j < C; ++j) sCK[j * LD + c] = cacc[j];
  __syncthreads();

  // ---- element terms for this thread's rows
  const float gC = sG[(C - 1) * LD + c];
  const E* gdQL = static_cast<const E*>(p.dQL) + (size_t)rec * C * D;
  const E* gdKt = static_cast<const E*>(p.dKt) + (size_t)rec * C * D;
  const E* gdBk = static_cast<const E*>(p.dBk) + (size_t)rec * C * D;
  const E* gdBv = static_cast<const E*>(p.dBv) + (size_t)rec * C * D;
  float colsum = 0.f;  // sum over this thread's rows of dKt Ktil
  float dgam[4][4], dbp[4][4];
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * ck[m] + r;
      const size_t lo = (size_t)t * D + c;
      const float dql = to_f32(gdQL[lo]), dkt = to_f32(gdKt[lo]), dbk = to_f32(gdBk[lo]),
                  dbv = to_f32(gdBv[lo]);
      const float kk = sK[t * LD + c], qq = sQ[t * LD + c], bt = sB[t];
      const float lam = __builtin_amdgcn_exp2f(sG[t * LD + c]);
      const float ec = __builtin_amdgcn_exp2f(gC - sG[t * LD + c]);
      const float ckt = sCK[t * LD + c];
      const float ktil = kk * ec;
      colsum = fmaf(dkt, ktil, colsum);
      dgam[m][r] = dbk * bt * kk * lam + dql * qq * lam - dkt * ktil + bt * kk * rK[m][r] +
                   qq * rQ[m][r] - kk * ckt;
      float vv = 0.f;
      if (t < nval) {
        const size_t o = row_of(t) + c;
        vv = to_f32(static_cast<const E*>(p.y)[2 * plane + o]);
        E* dy = static_cast<E*>(p.dy);
        dy[o] = from_f32<E>(lam * dql + rQ[m][r]);
        dy[plane + o] = from_f32<E>(bt * lam * dbk + ec * dkt + bt * rK[m][r] + ckt);
        dy[2 * plane + o] = from_f32<E>(bt * dbv);
      }
      dbp[m][r] = dbv * vv + dbk * kk * lam + kk * rK[m][r];
    }
  }
  colsum = group_sum<TPC>(colsum);
  __syncthreads();  // every read of cK and Q is done
  float* sdG = sQ;   // [C][LD]
  float* sdb = sAP;  // [C][LD]
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * ck[m] + r;
      sdG[t * LD + c] = dgam[m][r];
      sdb[t * LD + c] = dbp[m][r];
    }
  if (tq == 0) sGC[c] = colsum + p.dLC[(size_t)rec * D + c] * __builtin_amdgcn_exp2f(gC);
  __syncthreads();
  // dg: reverse running sum over the chunk, one thread per channel
  if (tid < D) {
    float acc = sGC[tid];
    for (int t = C - 1; t >= 0; --t) {
      acc += sdG[t * LD + tid];
      if (t < nval) p.dg[row_of(t) + tid] = acc;
    }
  }
  // dbeta: sum over the channels, one thread per token
  if (tid < nval) {
    float acc = 0.f;
    for (int cc = 0; cc < D; ++cc) acc += sdb[tid * LD + cc];
    p.dbeta_part[((size_t)rt.tok + tid) * p.H + h] = acc;
  }
}

// ------------------------------------------------------- front end in reverse
// One 256-thread workgroup per (b, h, block of TOKB = 4 * 256 / (D / 8) tokens);
// a thread owns 4 tokens x 8 channels and the D / 8 lanes of a token row reduce
// the L2 sums together.  For each of q, k, v, with pre the conv output, y =
// SiLU(pre) and z = y / n, n = sqrt(|y|^2 + eps) (q and k):
//   dy = dz / n - y (y . dz) / n^3,   dpre = dy sigmoid(pre) (1 + pre (1 - sigmoid(pre)))
//   dx_t = sum_tau w_tau dpre_{t + 3 - tau},   dw_tau = sum_t dpre_t x_{t - 3 + tau}
// dpre of the block goes through LDS; the last segment also forms it for the 3
// tokens after the block (the conv reaches them).  Tokens before the sequence
// take their raw values from the conv history (their gradient goes to
// dconv_state).  The filter partials are summed over the lanes of a wave, then
// over the waves, in a fixed order.  dbeta (summed by the pair kernel) is copied.
template <int D, typename IO>
__global__ __launch_bounds__(256, 2) void kda_bwd_front_kernel(BwdFrontParams p, const float* dbeta_part,
                                                               int nparts, float* dbeta) {
  constexpr int NOCT = D / 8;
  constexpr int SEG = 256 / NOCT;
  constexpr int TOKB = 4 * SEG;  // tokens per workgroup
  constexpr int LDP = D + 4;
  constexpr int SPW = 64 / NOCT;  // segments per wave
  constexpr int NW = 4;           // waves
  static_assert(SPW >= 3, "the last wave holds the 3 segments that take the rows past the block");
  __shared__ float sw[3 * 4 * D];            // filters [x][tap][c]
  __shared__ float sdp[(TOKB + 3) * LDP];    // dpre of the block and the 3 tokens after it
  __shared__ float sred[4][3 * 4 * D];       // filter partials per wave [x][tap][c]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t HD = (size_t)p.H * D;
  // the workgroup's sequence b, head h, block of the sequence, the sequence's
  // first token row and length, and the slot of its filter partial.  Block-major
  // order: the workgroups running at the same time cover every head of a few
  // token blocks, so together they read and write whole token rows (all heads of
  // a token are adjacent in memory) instead of one head's slice of many rows.
  int h, b, blk, Tq, part;
  long tok0;
  if (p.seqs.bounds == nullptr) {
    const int nblk = (p.T + TOKB - 1) / TOKB;
    const int BH = p.B * p.H;
    blk = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    h = bh % p.H;
    b = bh / p.H;
    Tq = p.T;
    tok0 = (long)b * p.T;
    part = b * nblk + blk;
  } else {
    part = blockIdx.x / p.H;
    h = blockIdx.x % p.H;
    const bool used = part < p.fstart[p.seqs.n_seqs];
    b = used ? seq_of_slot(p.fstart, p.seqs.n_seqs, part) : 0;
    blk = used ? part - p.fstart[b] : 0;
    tok0 = used ? p.seqs.bounds[b] : 0;
    Tq = used ? p.seqs.bounds[b + 1] - p.seqs.bounds[b] : 0;
    if (!used || blk * TOKB >= Tq) {
      // a slot no sequence uses: its filter partial is zero
      if (p.conv_w != nullptr)
        for (int it = tid; it < 3 * 4 * D; it += 256) {
          const int x = it / (4 * D), tau = (it / D) % 4, c = it % D;
          p.dconv_part[((size_t)part * 3 + x) * HD * 4 + ((size_t)h * D + c) * 4 + tau] = 0.f;
        }
      return;
    }
  }
  const int s = tid / NOCT, j = tid % NOCT;
  const int ch = 8 * j;
  const int t0 = blk * TOKB;
  const int tf = t0 + 4 * s;
  const size_t plane = (size_t)p.B * p.T * HD;
  const bool conv = p.conv_w != nullptr;
  if (conv)
    for (int it = tid; it < 3 * D; it += 256) {
      const int x = it / D, c = it % D;
      const f32x4 w = *reinterpret_cast<const f32x4*>(p.conv_w + ((size_t)x * HD + (size_t)h * D + c) * 4);
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) sw[(x * 4 + tau) * D + c] = w[tau];
    }
  __syncthreads();

  for (int x = 0; x < 3; ++x) {
    const IO* src = x == 0 ? static_cast<const IO*>(p.q) : (x == 1 ? static_cast<const IO*>(p.k)
                                                                   : static_cast<const IO*>(p.v));
    float* dst = x == 0 ? p.dq : (x == 1 ? p.dk : p.dv);
    // Every global load of this tensor is issued before the first use, as
    // range-checked buffer loads (zeros outside the range, no branches between
    // the loads): raw rows t_first - 3 .. t_first + 3 (row m = token t_first - 3 + m;
    // tokens < 0 from the conv history) and the rows of dz for tokens t_first ..
    // t_first + 3.  The dx of the block's last tokens also needs the dpre of the 3
    // tokens past the block: in the last wave, segment SEG - SPW + hh (hh < 3)
    // computes token t0 + TOKB + hh for its channels, from raw rows of that token
    // and 3 before it and its dz row (so no wave takes more than 5 rows).  The
    // workgroup's rows are [max(t0 - 3, 0), min(t0 + TOKB + 3, T)).
    const int hh = s - (SEG - SPW);                     // 0 .. SPW - 1 in the last wave
    const bool halo = hh >= 0 && hh < 3;
    const int hc = halo ? hh : 0;                       // a valid row for the others' loads
    Raw8<IO> rw[7], hw[4];
    Raw8<IO> dzr[4], hz;
    {
      constexpr int ES = (int)sizeof(IO);
      const int r0 = t0 - 3 > 0 ? t0 - 3 : 0;
      const int r1 = t0 + TOKB + 3 < Tq ? t0 + TOKB + 3 : Tq;
      const int row_b = (int)(HD * ES);
      const BufRes rx = make_buf(src + ((size_t)tok0 + r0) * HD + (size_t)h * D,
                                 (unsigned)(((long)(r1 - 1 - r0) * HD + D) * ES));
      const int voff = (tf - 3 - r0) * row_b + ch * ES;
#pragma unroll
      for (int m = 0; m < 7; ++m) rw[m].load(rx, voff + m * row_b, 0);
      const int hoff = (t0 + TOKB + hc - 3 - r0) * row_b + ch * ES;
#pragma unroll
      for (int m = 0; m < 4; ++m) hw[m].load(rx, hoff + m * row_b, 0);
      const int rz1 = t0 + TOKB + 3 < Tq ? t0 + TOKB + 3 : Tq;
      const BufRes rz = make_buf(static_cast<const IO*>(p.dy) + x * plane + ((size_t)tok0 + t0) * HD +
                                     (size_t)h * D,
                                 (unsigned)(((long)(rz1 - 1 - t0) * HD + D) * ES));
      const int zoff = (tf - t0) * row_b + ch * ES;
#pragma unroll
      for (int u = 0; u < 4; ++u) dzr[u].load(rz, zoff + u * row_b, 0);
      hz.load(rz, (TOKB + hc) * row_b + ch * ES, 0);
      if (conv && p.conv_state_in != nullptr && t0 == 0) {
        // tokens -3 .. -1 sit in history rows 0 .. 2 (only the first segment reaches them)
        const BufRes rs = make_buf(static_cast<const IO*>(p.conv_state_in) + ((size_t)b * 3 + x) * 3 * HD +
                                       (size_t)h * D,
                                   (unsigned)((2 * HD + D) * ES));
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          Raw8<IO> sv;
          sv.load(rs, (tf + m) * row_b + ch * ES, 0);  // history row tf + m = token tf - 3 + m
          rw[m].merge(sv);
        }
      }
    }
    float raw[7][8];
#pragma unroll
    for (int m = 0; m < 7; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) raw[m][c] = rw[m][c];
    float w[4][8];
    if (conv) {
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int c = 0; c < 8; ++c) w[tau][c] = sw[(x * 4 + tau) * D + ch + c];
    }
    // dpre of one token into sdp row srow, from the raw rows rr[u0 .. u0 + 3] (the
    // token and the 3 before it) and its dz row
    auto dpre_row = [&](const auto& rr, int u0, const Raw8<IO>& dzrow, int srow, bool st) {
      // sigmoid(pre) once per element, with the hardware exp2 and reciprocal as in
      // the forward front end (so y is the forward's value), for y = pre sigmoid(pre)
      // and for the SiLU derivative
      float pre[8], sg[8], y[8], dz[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (conv) {
          float acc = w[0][c] * rr[u0][c];
          acc = fmaf(w[1][c], rr[u0 + 1][c], acc);
          acc = fmaf(w[2][c], rr[u0 + 2][c], acc);
          acc = fmaf(w[3][c], rr[u0 + 3][c], acc);
          pre[c] = acc;
          sg[c] = sigmoid_fast(acc);
          y[c] = acc * sg[c];
        } else {
          pre[c] = 0.f;
          sg[c] = 1.f;
          y[c] = rr[u0 + 3][c];
        }
        dz[c] = dzrow[c];  // zero past the end of the sequence
        if (x == 0) dz[c] *= p.scale;
      }
      float dyv[8];
      if (x < 2 && p.l2) {
        float yy = 0.f, yd = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          yy = fmaf(y[c], y[c], yy);
          yd = fmaf(y[c], dz[c], yd);
        }
        yy = group_sum<NOCT>(yy);
        yd = group_sum<NOCT>(yd);
        const float rn = __builtin_amdgcn_rsqf(yy + p.eps);  // as the forward normalises
        const float k3 = yd * rn * rn * rn;
#pragma unroll
        for (int c = 0; c < 8; ++c) dyv[c] = dz[c] * rn - y[c] * k3;
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) dyv[c] = dz[c];
      }
      float dp[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (conv) {
          dp[c] = dyv[c] * sg[c] * (1.0f + pre[c] * (1.0f - sg[c]));
        } else {
          dp[c] = dyv[c];
        }
      }
      if (st) {
        *reinterpret_cast<f32x4*>(&sdp[srow * LDP + ch]) = f32x4{dp[0], dp[1], dp[2], dp[3]};
        *reinterpret_cast<f32x4*>(&sdp[srow * LDP + ch + 4]) = f32x4{dp[4], dp[5], dp[6], dp[7]};
      }
    };
#pragma unroll
    for (int u = 0; u < 4; ++u) dpre_row(raw, u, dzr[u], 4 * s + u, true);
    if (wave == NW - 1) {  // the whole wave takes this branch
      float hraw[4][8];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) hraw[m][c] = hw[m][c];
      dpre_row(hraw, 0, hz, TOKB + hc, halo);
    }
    __syncthreads();
    // dx of the own tokens
    float dpo[7][8];
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(&sdp[(4 * s + u) * LDP + ch]);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(&sdp[(4 * s + u) * LDP + ch + 4]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        dpo[u][c] = tf + u < Tq ? lo[c] : 0.f;
        dpo[u][c + 4] = tf + u < Tq ? hi[c] : 0.f;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = tf + m;
      if (t < Tq) {
        float dx[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (conv)
            dx[c] = w[3][c] * dpo[m][c] + w[2][c] * dpo[m + 1][c] + w[1][c] * dpo[m + 2][c] +
                    w[0][c] * dpo[m + 3][c];
          else
            dx[c] = dpo[m][c];
        }
        store8(dst + ((size_t)tok0 + t) * HD + (size_t)h * D + ch, dx);
      }
    }
    if (conv) {
      // gradient of the conv history (tokens -3 .. -1) from the first segment
      if (tf == 0 && p.dconv_state != nullptr) {
#pragma unroll
        for (int u = -3; u < 0; ++u) {
          float dx[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
              const int tt = u + 3 - tau;  // token whose window holds token u at tap tau
              if (tt >= 0) acc = fmaf(w[tau][c], dpo[tt][c], acc);
            }
            dx[c] = acc;
          }
          store8(p.dconv_state + (((size_t)b * 3 + x) * 3 + (3 + u)) * HD + (size_t)h * D + ch, dx);
        }
      }
      // filter partials of the own tokens, summed over the wave's segments
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m) acc = fmaf(dpo[m][c], raw[m + tau][c], acc);
#pragma unroll
          for (int o = NOCT; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
          if (lane < NOCT) sred[wave][(x * 4 + tau) * D + ch + c] = acc;
        }
    }
    __syncthreads();  // sdp is rewritten by the next tensor
  }
  if (conv) {
    for (int it = tid; it < 3 * 4 * D; it += 256) {
      const int x = it / (4 * D), tau = (it / D) % 4, c = it % D;
      const float acc = sred[0][it] + sred[1][it] + sred[2][it] + sred[3][it];
      p.dconv_part[((size_t)part * 3 + x) * HD * 4 + ((size_t)h * D + c) * 4 + tau] = acc;
    }
  }
  if (dbeta != nullptr && j == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = tf + m;
      if (t < Tq) {
        const size_t o = ((size_t)tok0 + t) * p.H + h;
        float acc = 0.f;
        for (int q = 0; q < nparts; ++q) acc += dbeta_part[(size_t)q * p.B * p.T * p.H + o];
        dbeta[o] = acc;
      }
    }
  }
}

// Clears the count of chunks listed for the exact pair kernel.
__global__ void kda_bwd_clear_kernel(unsigned* count) {
  if (threadIdx.x == 0) *count = 0u;
}

// dconv_w = the sum of the workgroups' partials (fixed order: deterministic)
__global__ __launch_bounds__(256) void kda_bwd_conv_reduce_kernel(const float* part, float* out,
                                                                  size_t n, int nparts) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  float acc = 0.f;
  // eight loads in flight ahead of their (in-order) adds
#pragma unroll 8
  for (int q = 0; q < nparts; ++q) acc += part[(size_t)q * n + idx];
  out[idx] = acc;
}

// ------------------------------------------------------------------ launchers
template <int D, int C, typename IO, typename E>
static hipError_t launch_bwd_t(const BwdLaunch& L, hipStream_t st) {
  // records (packed: one row of tokens, H * NT slots); walks per (sequence, head)
  const size_t nrec = (size_t)L.prod.B * L.prod.H * L.prod.NT;
  const size_t BH = (size_t)L.walk.B * L.walk.H;
  // reverse walk, one workgroup per value block of 64 columns (of D when D < 64);
  // split: the segments' reverse maps, their composition, the segment walks
  constexpr bool WIDE = D == 128 && sizeof(E) == 2;
  constexpr int WVB = WIDE ? 64 : (D >= 64 ? 64 : D);
  constexpr int WNT = WIDE ? 512 : 256;
  const size_t walks = BH * (D / WVB);
  if (L.walk.nseg > 1) {
    hipLaunchKernelGGL((kda_bwd_walk_kernel<D, C, WVB, IO, E, WNT, true>),
                       dim3((unsigned)(walks * (L.walk.nseg - 1))), dim3(WNT), 0, st, L.walk);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    SplitParams q{};
    q.S0 = L.walk.dS_T;
    q.maps = L.walk.maps;
    q.starts = L.walk.starts;
    q.B = L.walk.B; q.H = L.walk.H; q.NT = L.walk.NT;
    q.nseg = L.walk.nseg; q.seg_len = L.walk.seg_len;
    q.reverse = 1;
    if (hipError_t e = launch_split_combine(q, D, st); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((kda_bwd_walk_kernel<D, C, WVB, IO, E, WNT, false>),
                     dim3((unsigned)(walks * (L.walk.nseg > 1 ? L.walk.nseg : 1))), dim3(WNT), 0, st,
                     L.walk);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((kda_bwd_prod_kernel<D, C, IO, E>), dim3((unsigned)nrec), dim3(256), 0, st, L.prod);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if constexpr (sizeof(E) == 2) {
    hipLaunchKernelGGL((kda_bwd_t16_kernel<D, C>), dim3((unsigned)nrec), dim3(512), 0, st, L.tside);
  } else {
    // persistent: as many workgroups as fit on the device at once
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kda_bwd_t_kernel<D, C, E>, 512, 0) != hipSuccess)
      return hipErrorInvalidValue;
    const size_t fit = (size_t)(per > 0 ? per : 1) * (size_t)(cus > 0 ? cus : 1);
    hipLaunchKernelGGL((kda_bwd_t_kernel<D, C, E>), dim3((unsigned)(nrec < fit ? nrec : fit)), dim3(512), 0,
                       st, L.tside);
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  constexpr int NBLK = 1;  // the pair kernels sum dbeta over all channels themselves
  // factored products for every chunk; the exact kernel takes the ones they list
  hipLaunchKernelGGL(kda_bwd_clear_kernel, dim3(1), dim3(64), 0, st, L.pair.ex_count);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((kda_bwd_pair_mma_kernel<D, C, E>), dim3((unsigned)nrec), dim3(4 * D), 0, st, L.pair);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  constexpr int PNTH = PairShape<D, C>::NTH;
  hipLaunchKernelGGL((kda_bwd_pair_kernel<D, C, E>), dim3((unsigned)nrec), dim3(PNTH), 0, st, L.pair);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  constexpr int TOKB = 4 * (256 / (D / 8));
  const size_t nblk = ((size_t)L.front.T + TOKB - 1) / TOKB;
  // filter partials: one per (sequence, block) slot
  const size_t nparts = L.front.seqs.bounds != nullptr ? (size_t)L.front.nfslots : (size_t)L.front.B * nblk;
  hipLaunchKernelGGL((kda_bwd_front_kernel<D, IO>), dim3((unsigned)(L.front.H * nparts)), dim3(256), 0, st,
                     L.front, L.pair.dbeta_part, NBLK, L.dbeta);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (L.front.conv_w != nullptr) {
    const size_t n = (size_t)3 * L.front.H * D * 4;
    hipLaunchKernelGGL(kda_bwd_conv_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       L.front.dconv_part, L.dconv_w, n, (int)nparts);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, typename IO, typename E>
static hipError_t launch_bwd_c(const BwdLaunch& L, int C, hipStream_t st) {
  switch (C) {
    case 16: return launch_bwd_t<D, 16, IO, E>(L, st);
    case 32: return launch_bwd_t<D, 32, IO, E>(L, st);
    case 64:
      // fp32 at D = 128 takes C <= 32 (the product kernel's staged tiles need more
      // threads than it has at C = 64; the forward rejects that chunk size too)
      if constexpr (D == 128 && sizeof(E) == 4) return hipErrorInvalidValue;
      else return launch_bwd_t<D, 64, IO, E>(L, st);
  }
  return hipErrorInvalidValue;
}

size_t bwd_front_blocks(int T, int D) { return ((size_t)T + 4 * (256 / (D / 8)) - 1) / (4 * (256 / (D / 8))); }
int bwd_front_tokens(int D) { return 4 * (256 / (D / 8)); }

hipError_t launch_backward(const BwdLaunch& L, int D, int C, bool fp32, hipStream_t st) {
  if (fp32) {
    switch (D) {
      case 16: return launch_bwd_c<16, float, float>(L, C, st);
      case 32: return launch_bwd_c<32, float, float>(L, C, st);
      case 64: return launch_bwd_c<64, float, float>(L, C, st);
      case 128: return launch_bwd_c<128, float, float>(L, C, st);
    }
  } else {
    switch (D) {
      case 16: return launch_bwd_c<16, __bf16, __bf16>(L, C, st);
      case 32: return launch_bwd_c<32, __bf16, __bf16>(L, C, st);
      case 64: return launch_bwd_c<64, __bf16, __bf16>(L, C, st);
      case 128: return launch_bwd_c<128, __bf16, __bf16>(L, C, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
