// State walk of the KDA prefill: one workgroup (4 or 8 waves) per (sequence,
// head, block of VB value columns), walking the chunks of the sequence in order.
// Value columns of the state evolve independently (every product below is
// column-wise in v), so splitting them across workgroups is exact and gives
// B*H*(D/VB) parallel walks.
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
// The chunk record is copied into LDS by the asynchronous global-to-LDS loads of
// gfx950 (16 bytes per lane straight into LDS, no registers involved).  Each
// chunk's fragments are read from LDS into registers at the start of its step,
// after which the copy of the next chunk is issued and runs under the step's
// arithmetic.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace kda {


// 4 consecutive elements kept raw until used
template <typename E> struct Raw4;
template <> struct Raw4<__bf16> {
  bf16x4 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const bf16x4*>(p); }
  __device__ __forceinline__ float operator[](int i) const { return (float)v[i]; }
};
template <> struct Raw4<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ float operator[](int i) const { return v[i]; }
};

// The LDS image of the part of one chunk record a workgroup reads.  Byte offsets;
// every part is a whole number of 16-byte chunks.
template <int D, int C, int VB, typename E>
struct RecImage {
  static constexpr int ES = (int)sizeof(E);
  static constexpr int W = 0;                          // [C][D] swizzled
  static constexpr int QL = W + C * D * ES;            // [C][D] swizzled
  static constexpr int KT = QL + C * D * ES;           // [D][C] swizzled
  static constexpr int P = KT + D * C * ES;            // [C][C] swizzled
  static constexpr int U = P + C * C * ES;             // (C/16) x (VB/16) fragment tiles
  static constexpr int LC = U + C * VB * ES;           // [D] float
  static constexpr int BYTES = LC + D * 4;
  static constexpr int CHUNKS = BYTES / 16;
  static_assert(BYTES % 16 == 0, "record image is whole 16-byte chunks");
};

// GN: apply the output stage (RMSNorm with gain over the head's D values, sigmoid
// gate) before storing o.  Only with VB == D, where one workgroup holds every
// value column of its tokens.
template <int D, int C, int VB, typename IO, typename E, int NT, bool GN, bool CK>
__global__ __launch_bounds__(NT, NT == 256 ? 2 : 1) void kda_chunk_state_kernel(StateParams p) {
  static_assert(!GN || VB == D, "the output stage needs whole rows");
  constexpr int NW = NT / 64;  // waves
  constexpr int PE = 16 / (int)sizeof(E);
  constexpr int ES = (int)sizeof(E);
  constexpr int LS = D + PE;  // sS row stride: row = value column v, k = key channel c
  constexpr int LU = C + PE;  // sU row stride: row = value column v, k = token t
  constexpr int NV = D / VB;
  constexpr int VT = VB / 16;   // v-tiles
  constexpr int RT = C / 16;    // t-tiles
  constexpr int CT = D / 16;    // c-tiles
  static_assert(NW % RT == 0, "every unit of a wave has the same t-tile");
  static_assert(CT <= NW || CT % NW == 0, "every unit of a wave has one of NCTW c-tiles");
  constexpr int NU = (RT * VT + NW - 1) / NW;  // (t-tile, v-tile) units per wave (upper bound)
  constexpr int NS = (CT * VT + NW - 1) / NW;  // (c-tile, v-tile) units per wave (upper bound)
  constexpr int CTW = CT < NW ? CT : NW;       // c-tile stride between a wave's units
  constexpr int NCTW = CT > NW ? CT / NW : 1;  // distinct c-tiles per wave
  constexpr bool FULL_U = (RT * VT) % NW == 0;
  constexpr bool FULL_S = (CT * VT) % NW == 0;
  constexpr RecordLayout RL = record_layout(C, D, sizeof(E));
  using IMG = RecImage<D, C, VB, E>;
  __shared__ __attribute__((aligned(16))) char img[IMG::BYTES];
  __shared__ __attribute__((aligned(16))) E sS[VB * LS];
  __shared__ __attribute__((aligned(16))) E sU[VB * LU];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  // Workgroups of one head's value blocks are placed on the same XCD (dispatch
  // is round robin over the 8 XCDs), so they share the chunk records in L2.
  int bh, vblk, seg = 0;
  if (p.nseg > 1) {
    // split walk: (head, segment) groups of NV workgroups, numbered XCD by XCD
    const int grp = xcd_major(blockIdx.x, gridDim.x);
    vblk = grp % NV;
    bh = grp / NV % (p.B * p.H);
    seg = grp / NV / (p.B * p.H);
  } else if ((p.B * p.H * NV) % (8 * NV) == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    vblk = slot % NV;
    bh = (slot / NV) * 8 + xcd;
  } else {
    vblk = blockIdx.x % NV;
    bh = blockIdx.x / NV;
  }
  const int h = bh % p.H, b = bh / p.H;
  const int vb0 = vblk * VB;
  // This walk's tokens and records: sequence b of B equal-length ones, or packed
  // sequence b (tokens [bounds[b], bounds[b + 1]), chunk slots from cstart[b] of
  // head h).
  // Chunk n of this walk is record rec0 + n rstride (rec_slot).
  long tok0;
  int Tq, nch;
  size_t rec0, rstride;
  if (p.seqs.bounds == nullptr) {
    // chunks c0 .. of sequence b: tokens from c0 C on, at most cap chunks (a
    // time slice's records fill the workspace from slot 0; a segment's are
    // slots c0 .. of the sequence's)
    const int c0 = p.nseg > 1 ? seg * p.seg_len : p.c0;
    const int cap = p.nseg > 1 ? p.seg_len : p.NT;
    tok0 = (long)b * p.T + (long)c0 * C;
    Tq = p.T - c0 * C;
    nch = (Tq + C - 1) / C < cap ? (Tq + C - 1) / C : cap;
    rstride = (size_t)p.B * p.H;
    rec0 = rec_slot(p.nseg > 1 ? c0 : 0, bh, rstride);
  } else {
    tok0 = p.seqs.bounds[b];
    Tq = p.seqs.bounds[b + 1] - p.seqs.bounds[b];
    // slots clamped to this head's NT, so the records read stay in the workspace
    int c0 = p.seqs.cstart[b], c1 = p.seqs.cstart[b + 1];
    c0 = c0 < 0 ? 0 : (c0 > p.NT ? p.NT : c0);
    c1 = c1 < c0 ? c0 : (c1 > p.NT ? p.NT : c1);
    nch = c1 - c0;
    rstride = (size_t)p.H;
    rec0 = rec_slot(c0, h, rstride);
  }
  // conv-state hand-over of (b, h): new state row tau = raw input at position
  // Tq - 3 + tau, from the previous state where that position is < 0.  A thread
  // reads the 3 values of its (tensor, channel) before writing them, so the new
  // state may overwrite the previous one.
  if (p.tail_out != nullptr && vblk == 0 && seg == 0) {
    const size_t HD = (size_t)p.H * D;
    for (int it = tid; it < 3 * D; it += NT) {
      const int i = it / D;
      const size_t col = (size_t)h * D + it % D;
      const IO* x = static_cast<const IO*>(i == 0 ? p.tail_x[0] : (i == 1 ? p.tail_x[1] : p.tail_x[2]));
      const IO* in = static_cast<const IO*>(p.tail_in);
      IO* out = static_cast<IO*>(p.tail_out) + ((size_t)b * 3 + i) * 3 * HD + col;
      IO val[3];
#pragma unroll
      for (int tau = 0; tau < 3; ++tau) {
        const int t = Tq - 3 + tau;
        if (t >= 0)
          val[tau] = x[((size_t)tok0 + t) * HD + col];
        else if (in != nullptr)
          val[tau] = in[((size_t)b * 3 + i) * 3 * HD + (size_t)(3 + t) * HD + col];
        else
          val[tau] = from_f32<IO>(0.f);
      }
#pragma unroll
      for (int tau = 0; tau < 3; ++tau) out[(size_t)tau * HD] = val[tau];
    }
  }

  // this wave's tiles
  const int R = wave % RT;                      // t-tile of every (t, v) unit of this wave
  const bool has_u = FULL_U || wave < RT * VT;  // any (t, v) unit at all
  const int i_row = 16 * R + r;                 // row of P / W / QL this lane reads
  const int csteps = (16 * R + 16 + RowFrag<E, C>::STEP - 1) / RowFrag<E, C>::STEP;

  // ---- asynchronous copy of a chunk's record image into LDS.  Thread tid moves
  // 16-byte chunk it * 256 + tid of the image; its source offset inside the
  // record is the same for every chunk, so it is computed once.
  constexpr int ITERS = (IMG::CHUNKS + NT - 1) / NT;
  uint32_t src_off[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    constexpr int RCD = D * ES / 16;           // chunks per row of W, QL
    constexpr int RCC = C * ES / 16;           // chunks per row of KT, P
    constexpr int UPIECE = VT * 64 * 4 * ES / 16;  // chunks of U~ per t-tile: VT tiles x 64 lanes x 4
    const int idx = it * NT + tid;
    const int byte = idx * 16;
    size_t off;
    if (byte < IMG::KT) {
      // W or QL: rows of RCD chunks, stored swizzled
      const bool isql = byte >= IMG::QL;
      const int ci = idx - (isql ? IMG::QL / 16 : 0);
      const int row = ci / RCD, cs = ci % RCD;
      off = (size_t)(isql ? RL.ql : RL.w) * ES + (size_t)(row * RCD + (cs ^ (row & (RCD - 1)))) * 16;
    } else if (byte < IMG::U) {
      // KT or P: rows of RCC chunks, stored swizzled
      const bool isp = byte >= IMG::P;
      const int ci = idx - (isp ? IMG::P : IMG::KT) / 16;
      const int row = ci / RCC, cs = ci % RCC;
      off = (size_t)(isp ? RL.p : RL.kt) * ES + (size_t)(row * RCC + (cs ^ (row & (RCC - 1)))) * 16;
    } else if (byte < IMG::LC) {
      // U~ tiles of this value block, one contiguous piece per t-tile
      const int ci = idx - IMG::U / 16;
      const int tt = ci / UPIECE, w = ci % UPIECE;
      off = (size_t)RL.u * ES + ((size_t)(tt * (D / 16) + vb0 / 16) * 64 * 4) * ES + (size_t)w * 16;
    } else {
      off = RL.lc_bytes + (size_t)(idx - IMG::LC / 16) * 16;
    }
    src_off[it] = (uint32_t)off;
  }
  auto issue_copy = [&](int n) {
    const char* recp = p.ws + (rec0 + n * rstride) * RL.bytes;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      // this wave's 64 lanes fill img + (it * NT + 64 * wave) * 16 onwards, 16 bytes per lane
      if (it * NT + tid < IMG::CHUNKS)
        __builtin_amdgcn_global_load_lds(
            (const glb_void_t*)(recp + src_off[it]),
            (lds_void_t*)(img + (size_t)(it * NT + 64 * wave) * 16), 16, 0, 0);
    }
  };

  // ---- initial state (a segment's from the composed start states; S_T, which
  // may be S0, is written by the last segment only)
  f32x4 accS[NS];
  const size_t sbase = (size_t)bh * D * D;
  const float* s_in = p.nseg > 1 ? p.seg_start + ((size_t)bh * p.nseg + seg) * D * D
                                 : (p.S0 != nullptr ? p.S0 + sbase : nullptr);
  float* s_out = p.nseg > 1 && seg != p.nseg - 1 ? nullptr
                 : (p.S_T != nullptr ? p.S_T + sbase : nullptr);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = wave + NW * i;
    accS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if ((FULL_S || u < CT * VT) && s_in != nullptr) {
      const int Ct = u % CT, Vt = u / CT;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        accS[i][e] = s_in[(size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r];
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

  IO* o = static_cast<IO*>(p.o);
  const size_t HD = (size_t)p.H * D;
  const E* iW = reinterpret_cast<const E*>(img + IMG::W);
  const E* iQL = reinterpret_cast<const E*>(img + IMG::QL);
  const E* iKT = reinterpret_cast<const E*>(img + IMG::KT);
  const E* iP = reinterpret_cast<const E*>(img + IMG::P);
  const E* iU = reinterpret_cast<const E*>(img + IMG::U);
  const float* iLC = reinterpret_cast<const float*>(img + IMG::LC);

  // The output of chunk n is stored during step n + 1, after its U and S^T QL^T
  // products: by then the wave has issued the copy of chunk n + 2, so the stores
  // neither queue behind that copy nor delay the products, and they retire while
  // the rest of step n + 1 computes.
  f32x4 pendO[NU];
  // Output stage (GN): lane (r, g4) of a unit holds token 16 R + r and value rows
  // 16 Vt + 4 g4 + e.  Each wave leaves its per-token sums of squares of chunk n
  // in buffer n % 2 of ored (a wave of step n + 1 may write its sums before a
  // slower wave has read chunk n's); the waves of one t-tile are those with
  // wave % RT == R.  The gate rows of
  // chunk n are copied into buffer n % 2 of sgate at the start of step n, with
  // the record copy of chunk n + 1 (the same wait covers both), and read at the
  // store of chunk n in step n + 1.  A buffer holds [C][D] in 16-byte pieces,
  // piece c of row t at c ^ (t % GRP) (conflict-free reads of 16 rows at one
  // column).
  constexpr int GRP = D * (int)sizeof(IO) / 16;  // 16-byte pieces per gate row
  constexpr int GCH = C * GRP;                   // pieces per chunk
  __shared__ float ored[GN ? 2 * NW * 16 : 1];
  __shared__ __attribute__((aligned(16))) float onw[GN ? D : 1];  // norm gain (1 without norm)
  __shared__ __attribute__((aligned(16))) char sgate[GN ? 2 * GCH * 16 : 16];
  const bool has_norm = GN && p.o_norm_w != nullptr;
  const bool has_gate = GN && p.o_gate != nullptr;
  if constexpr (GN) {
    // visible to every wave after the loop's first barrier
    for (int c = tid; c < D; c += NT) onw[c] = has_norm ? p.o_norm_w[c] : 1.0f;
  }
  auto load_gate = [&](int nn) {
    if constexpr (GN) {
      if (!has_gate) return;
      const char* src = static_cast<const char*>(p.o_gate) +
                        (((size_t)tok0 + (size_t)nn * C) * HD + (size_t)h * D) * sizeof(IO);
#pragma unroll
      for (int it = 0; it < (GCH + NT - 1) / NT; ++it) {
        const int idx = it * NT + tid;
        const int tt = idx / GRP, cs = idx % GRP;
        // lanes of one wave fill 64 consecutive pieces from sgate + (it * NT + 64 * wave) * 16
        if (idx < GCH && nn * C + tt < Tq)
          __builtin_amdgcn_global_load_lds(
              (const glb_void_t*)(src + (size_t)tt * HD * sizeof(IO) + (size_t)((cs ^ (tt % GRP)) * 16)),
              (lds_void_t*)(sgate + (size_t)((nn & 1) * GCH + it * NT + 64 * wave) * 16), 16, 0, 0);
      }
    }
  };
  auto gate_at = [&](int nn, int tt, int v) {  // 4 gate values of chunk nn, row tt, columns v ..
    const int piece = v * (int)sizeof(IO) / 16, off = v * (int)sizeof(IO) % 16;
    Raw4<IO> gv;
    gv.load(reinterpret_cast<const IO*>(sgate + ((nn & 1) * GCH + tt * GRP + (piece ^ (tt % GRP))) * 16 + off));
    return gv;
  };
  auto row_sums = [&](int nn) {
    if constexpr (GN) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NU; ++i)
        if (FULL_U || wave + NW * i < RT * VT)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = fmaf(pendO[i][e], pendO[i][e], ss);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (g4 == 0) ored[((nn & 1) * NW + wave) * 16 + r] = ss;
    }
  };
  auto store_out = [&](int nn) {
    float rs = 1.f;
    if constexpr (GN) {
      if (has_norm) {
        float tot = 0.f;
#pragma unroll
        for (int w = R; w < NW; w += RT) tot += ored[((nn & 1) * NW + w) * 16 + r];
        rs = 1.0f / sqrtf(tot * (1.0f / D) + p.o_norm_eps);
      }
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (FULL_U || u < RT * VT) {
        const int Vt = u / RT;
        const int t = nn * C + 16 * R + r;
        f32x4 ov = pendO[i];
        if constexpr (GN) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(&onw[16 * Vt + 4 * g4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] *= rs * w[e];
          if (has_gate) {
            const Raw4<IO> gv = gate_at(nn, 16 * R + r, 16 * Vt + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] *= sigmoid(gv[e]);
          }
        }
        if (t < Tq)
          store4(o + ((size_t)tok0 + t) * HD + (size_t)h * D + vb0 + 16 * Vt + 4 * g4,
                 ov[0], ov[1], ov[2], ov[3]);
      }
    }
  };

  if (nch > 0) issue_copy(0);
  for (int n = 0; n < nch; ++n) {
    // this wave's copies of chunk n are done.  From step 2 on, the last vector
    // memory operations it issued are the NU output stores of chunk n - 2 (one per
    // unit, every token of a full chunk), issued after that copy: they may stay in
    // flight, as nothing in this kernel reads o.  (The output stage and the
    // checkpoints issue further operations, so those walks wait for everything.)
    if (!GN && !CK && n >= 2)
      wait_vmcnt<NU>();
    else
      __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // the whole image of chunk n and the state are in LDS
    // ---- this chunk's fragments, from the image into registers
    RowFrag<E, D> fw, fql;
    RowFrag<E, C> fp;
    RowFrag<E, C> fkt[NCTW];
    Raw4<E> fu[NU];
    f32x4 flc[NCTW];
    if (has_u) {
      load_swz<D>(fw, iW, i_row, g4);
      load_swz<D>(fql, iQL, i_row, g4);
      load_swz<C>(fp, iP, i_row, g4);
    }
#pragma unroll
    for (int j = 0; j < NCTW; ++j) {
      const int Ct = (wave % CTW) + CTW * j;
      load_swz<C>(fkt[j], iKT, 16 * Ct + r, g4);
      flc[j] = *reinterpret_cast<const f32x4*>(iLC + 16 * Ct + 4 * g4);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (FULL_U || u < RT * VT) fu[i].load(iU + ((size_t)(R * VT + u / RT) * 64 + lane) * 4);
    }
    lds_barrier();  // every wave holds its fragments: the image may be overwritten
    if (n + 1 < nch) issue_copy(n + 1);
    load_gate(n);  // buffer n % 2: chunk n - 2's, stored during step n - 1
    // backward mode: the record's checkpoint, S_n [c][v] then U [t][v].  Both are
    // written from their LDS copies (sS holds S_n as staged for this step, sU the
    // step's U after the next barrier): a lane reads 4 consecutive value columns of
    // one row there and stores them as one 4-element piece (the accumulators hold 4
    // rows of one column, which would take 4 scattered stores).
    E* ck = CK ? static_cast<E*>(p.ckpt) + (rec0 + n * rstride) * ((size_t)D * D + (size_t)C * D) : nullptr;
    if constexpr (CK) {
      constexpr int V4 = VB / 4;  // 4-column pieces per row of the block
#pragma unroll
      for (int k = 0; k < (D * V4 + NT - 1) / NT; ++k) {
        const int idx = tid + NT * k;
        if ((D * V4) % NT == 0 || idx < D * V4) {
          const int c = idx / V4, v4 = 4 * (idx % V4);
          store4(ck + (size_t)c * D + vb0 + v4, to_f32(sS[(v4) * LS + c]), to_f32(sS[(v4 + 1) * LS + c]),
                 to_f32(sS[(v4 + 2) * LS + c]), to_f32(sS[(v4 + 3) * LS + c]));
        }
      }
    }
    if (has_u) fp.mask_above(i_row, g4);

    // ---- U = U~ - W S  and  O^T = S^T QL^T
    f32x4 accO[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (FULL_U || u < RT * VT) {
        const int Vt = u / RT;
        RowFrag<E, D> sf;
        sf.load(sS + (16 * Vt + r) * LS, g4);
        f32x4 ws = {0.f, 0.f, 0.f, 0.f};
        mma<D>(ws, fw, sf);        // (t, v) tile of W S
        mma<D>(accO[i], sf, fql);  // (v, t) tile of S^T QL^T
        store4(&sU[(16 * Vt + r) * LU + 16 * R + 4 * g4], fu[i][0] - ws[0], fu[i][1] - ws[1],
               fu[i][2] - ws[2], fu[i][3] - ws[3]);
      }
    }
    lds_barrier();  // sU complete; every read of sS for this chunk is done
    if (n > 0) store_out(n - 1);
    if constexpr (CK) {
      // the same rounded U for the backward, from sU
      E* cu = ck + (size_t)D * D;
      constexpr int V4 = VB / 4;
#pragma unroll
      for (int k = 0; k < (C * V4 + NT - 1) / NT; ++k) {
        const int idx = tid + NT * k;
        if ((C * V4) % NT == 0 || idx < C * V4) {
          const int t = idx / V4, v4 = 4 * (idx % V4);
          store4(cu + (size_t)t * D + vb0 + v4, to_f32(sU[(v4) * LU + t]), to_f32(sU[(v4 + 1) * LU + t]),
                 to_f32(sU[(v4 + 2) * LU + t]), to_f32(sU[(v4 + 3) * LU + t]));
        }
      }
    }
    // ---- O^T += U^T P^T (j <= i), store O
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (FULL_U || u < RT * VT) {
        const int Vt = u / RT;
        RowFrag<E, C> uf;
        uf.load(sU + (16 * Vt + r) * LU, g4);
        mma<C>(accO[i], uf, fp, csteps);
        pendO[i] = accO[i];
      }
    }
    row_sums(n);
    // ---- S = Diag(Lambda_C) S + Ktil^T U
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (FULL_S || u < CT * VT) {
        const int Vt = u / CT;
        const int j = i % NCTW;  // this unit's c-tile is (wave % CTW) + CTW * j
        RowFrag<E, C> uf;
        uf.load(sU + (16 * Vt + r) * LU, g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[i][e] *= flc[j][e];
        mma<C>(accS[i], fkt[j], uf);
      }
    }
    stage_state();
  }
  if constexpr (GN) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gate copies
    lds_barrier();                  // the last chunk's row sums and gate rows
  }
  if (nch > 0) store_out(nch - 1);
  // ---- final state
  if (s_out != nullptr) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int u = wave + NW * i;
      if (FULL_S || u < CT * VT) {
        const int Ct = u % CT, Vt = u / CT;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s_out[(size_t)(16 * Ct + 4 * g4 + e) * D + vb0 + 16 * Vt + r] = accS[i][e];
      }
    }
  }
}

// One instantiation; CK (the backward mode's checkpoints) follows p.ckpt, so the
// forward walk carries no checkpoint code.
template <int D, int C, int VB, typename IO, typename E, int NT, bool GN>
static hipError_t launch_walk(const StateParams& p, size_t grid, hipStream_t st) {
  if (p.nseg > 1) grid *= (size_t)p.nseg;
  if (p.ckpt != nullptr) {
    if constexpr (GN) return hipErrorInvalidValue;  // no output stage in the backward mode
    else hipLaunchKernelGGL((kda_chunk_state_kernel<D, C, VB, IO, E, NT, false, true>),
                            dim3((unsigned)grid), dim3(NT), 0, st, p);
  } else {
    hipLaunchKernelGGL((kda_chunk_state_kernel<D, C, VB, IO, E, NT, GN, false>), dim3((unsigned)grid),
                       dim3(NT), 0, st, p);
  }
  return hipGetLastError();
}

template <int D, int C, typename IO, typename E>
static hipError_t launch_state_t(const StateParams& p, int vb, int threads, bool gn,
                                 hipStream_t st) {
  // vb value columns per workgroup (32 or 64, or D when D < 64); 512 threads only
  // with D = 128 and vb = 64.  gn (output stage in the walk) needs vb == D: 256
  // threads, D <= 64.
  const size_t BH = (size_t)p.B * p.H;
  if constexpr (D == 128) {
    if (!gn && vb == 64 && threads == 512) return launch_walk<D, C, 64, IO, E, 512, false>(p, BH * 2, st);
  }
  if (threads != 256) return hipErrorInvalidValue;
  if (gn) {
    if constexpr (D <= 64) {
      if (vb != D) return hipErrorInvalidValue;
      return launch_walk<D, C, D, IO, E, 256, true>(p, BH, st);
    }
    return hipErrorInvalidValue;
  }
  constexpr int VBmax = D >= 64 ? 64 : D;
  if (vb == 32 && D >= 32) {
    constexpr int VB = D >= 32 ? 32 : D;
    return launch_walk<D, C, VB, IO, E, 256, false>(p, BH * (D / VB), st);
  }
  return launch_walk<D, C, VBmax, IO, E, 256, false>(p, BH * (D / VBmax), st);
}

template <int D, typename IO, typename E>
static hipError_t launch_state_c(const StateParams& p, int C, int vb, int threads, bool gn,
                                 hipStream_t st) {
  switch (C) {
    case 16: return launch_state_t<D, 16, IO, E>(p, vb, threads, gn, st);
    case 32: return launch_state_t<D, 32, IO, E>(p, vb, threads, gn, st);
    case 64:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_state_t<D, 64, IO, E>(p, vb, threads, gn, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO, typename E>
static hipError_t launch_state_d(const StateParams& p, int D, int C, int vb, int threads, bool gn,
                                 hipStream_t st) {
  switch (D) {
    case 16: return launch_state_c<16, IO, E>(p, C, vb, threads, gn, st);
    case 32: return launch_state_c<32, IO, E>(p, C, vb, threads, gn, st);
    case 64: return launch_state_c<64, IO, E>(p, C, vb, threads, gn, st);
    case 128: return launch_state_c<128, IO, E>(p, C, vb, threads, gn, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state(const StateParams& p, int D, int C, bool fp32, int vb, int threads, bool gn,
                        hipStream_t st) {
  return fp32 ? launch_state_d<float, float>(p, D, C, vb, threads, gn, st)
              : launch_state_d<__bf16, __bf16>(p, D, C, vb, threads, gn, st);
}

// The output stage on its own, in place: one row of D values per (token, head),
// D / 8 threads per row, each with 8 consecutive values.  Used when the state
// walk splits a head's value columns over workgroups.
template <int D, typename IO>
__global__ __launch_bounds__(256) void kda_out_stage_kernel(OutStageParams p) {
  constexpr int G = D / 8;      // threads per row
  constexpr int RPW = 256 / G;  // rows per workgroup
  const long row = (long)blockIdx.x * RPW + threadIdx.x / G;
  const int j = threadIdx.x % G;
  const bool ok = row < p.rows;
  IO* o = static_cast<IO*>(p.o) + row * D + 8 * j;
  float x[8], gt[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = gt[c] = 0.f;
  if (ok) {
    load8(o, x);
    if (p.o_gate != nullptr) load8(static_cast<const IO*>(p.o_gate) + row * D + 8 * j, gt);
  }
  if (p.o_norm_w != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(x[c], x[c], ss);
    ss = group_sum<G>(ss);
    const float rs = 1.0f / sqrtf(ss * (1.0f / D) + p.o_norm_eps);
    float w[8];
    load8(p.o_norm_w + 8 * j, w);
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] *= rs * w[c];
  }
  if (p.o_gate != nullptr) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] *= sigmoid(gt[c]);
  }
  if (ok) store8(o, x);
}

template <typename IO>
static hipError_t launch_out_stage_t(const OutStageParams& p, int D, hipStream_t st) {
  const long rpw = 256 / (D / 8);
  const unsigned grid = (unsigned)((p.rows + rpw - 1) / rpw);
  switch (D) {
    case 16: hipLaunchKernelGGL((kda_out_stage_kernel<16, IO>), dim3(grid), dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL((kda_out_stage_kernel<32, IO>), dim3(grid), dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((kda_out_stage_kernel<64, IO>), dim3(grid), dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((kda_out_stage_kernel<128, IO>), dim3(grid), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_out_stage(const OutStageParams& p, int D, bool fp32, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  return fp32 ? launch_out_stage_t<float>(p, D, st) : launch_out_stage_t<__bf16>(p, D, st);
}

}  // namespace kda
