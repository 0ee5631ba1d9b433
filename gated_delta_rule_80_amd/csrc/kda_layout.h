// Workspace layout and kernel parameter blocks shared by the host runtime and
// the kernels.  No HIP types here: the host side includes it from plain C++.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// One workspace record per (sequence, head, chunk) holds what the chunk
// preparation hands to the state walk, in element type E (bf16 or fp32):
//   W      [C][D]  row-major   T diag(beta) (K * Lambda)
//   QL     [C][D]  row-major   scale * Q * Lambda
//   KT     [D][C]  row-major   (K * exp(Gamma_C - Gamma))^T
//   U      [C][D]  fragment order: tile (t/16, v/16) of 64 lanes x 4 values
//                  T diag(beta) V (the state-free part of the new values)
//   P      [C][C]  row-major   scale * (Q K^T masked, with relative decay), j <= i
//   LC     [D]     float32     exp(Gamma_C), the chunk's total decay
struct RecordLayout {
  size_t w, ql, kt, u, p;  // element offsets
  size_t lc_bytes;         // byte offset of LC
  size_t bytes;            // record size (256-byte multiple)
};

constexpr RecordLayout record_layout(int C, int D, size_t esize) {
  RecordLayout r{};
  const size_t cd = (size_t)C * D;
  r.w = 0;
  r.ql = cd;
  r.kt = 2 * cd;
  r.u = 3 * cd;
  r.p = 4 * cd;
  r.lc_bytes = round_up((4 * cd + (size_t)C * C) * esize, 16);
  r.bytes = round_up(r.lc_bytes + 4 * (size_t)D, 256);
  return r;
}

// Workspace: a 256-byte header whose first word counts the chunks the fast
// preparation handed to the exact one, the list of those chunk indices, for
// packed sequences their clamped token bounds and first chunk indices (int32,
// n_seqs + 1 each), then one record per (sequence, head, chunk) -- for packed
// sequences per (head, chunk slot), n_slots = ceil(T / C) + n_seqs slots a head.
// When the state walk is split into segments (below), their maps and start
// states follow the records.
//
// Records are chunk-major (rec_slot): a walk is one (sequence, head) pair,
// w = b H + h of NW = B H walks (packed sequences: w = h, NW = H, and the chunk
// index is the head's slot), and chunk n of walk w sits at slot n NW + w.  The
// walks step through their chunks together, so at any moment they read one
// contiguous stretch of records instead of NW stretches a whole head's records
// apart (equal low address bits, hence the same HBM channels); the preparation,
// whose workgroups run chunk by chunk over all heads, writes them the same way.
// Every per-record buffer of the backward uses the same slots.
constexpr size_t rec_slot(size_t n, size_t w, size_t nw) { return n * nw + w; }

struct WorkspaceLayout {
  size_t list;     // byte offset of the fallback list (uint32 per chunk)
  size_t seq;      // byte offset of the sequence tables (packed sequences)
  size_t records;  // byte offset of the first record
  size_t split;    // byte offset of the segment maps and start states
  size_t bytes;    // total
};

constexpr WorkspaceLayout workspace_layout(size_t nrec, int C, int D, size_t esize,
                                           size_t n_seqs = 0, size_t split_sz = 0) {
  WorkspaceLayout w{};
  w.list = 256;
  w.seq = round_up(w.list + 4 * nrec, 256);
  w.records = round_up(w.seq + (n_seqs > 0 ? 8 * (n_seqs + 1) : 0), 256);
  w.split = w.records + nrec * record_layout(C, D, esize).bytes;
  w.bytes = w.split + split_sz;
  return w;
}

// Split state walk.  The state after a run of chunks is affine in the state
// before it: S_end = M S_start + N, with M (D x D, acting on the key index) the
// product of the chunks' homogeneous maps S -> Diag(Lambda_C) S - Ktil^T W S and
// N the end state from zero.  The chunks of every (sequence, head) are cut into
// nseg segments of seg_len chunks (the last one shorter); each segment's N and M
// are walked in parallel, the segment start states are composed in order, and
// then every segment is walked with its outputs from its own start.
//   maps   [B*H][nseg - 1][3][D][D] float32, for segments s < nseg - 1: N
//          row-major [key][value] (for s = 0 walked from S0 itself, so it is the
//          state at the start of segment 1), then M transposed, Mt[j][c] =
//          M[c][j], then M row-major (the two M slots not written for s = 0);
//   starts [B*H][nseg][D][D] float32: the state at each segment's start.
// The reverse walk of the backward is affine in the same way: the gradient of a
// segment's start state is M^T (the gradient of its end state) + N', with N'
// the reverse walk of the segment from a zero end gradient (from dS_T for the
// last segment).  It reuses both buffers once the forward walk is done: N'_s in
// the N slot of segment s - 1 (s >= 1), and in starts[s] the gradient of the
// state at the end of segment s; reverse = 1 composes these from dS_T down.
// whole = 1 (the state map of a call): every segment's N (from zero, also for
// the first) and M, maps [B*H][nseg][3][D][D], the last segment nch - (nseg - 1)
// seg_len chunks long; the composition writes M and N of the whole call to
// M_out and N_out [B][H][D][D].
struct SplitParams {
  const char* ws;     // first record
  const float* S0;    // [B][H][D][D] or NULL (zeros); reverse: dS_T
  float* maps;
  float* starts;
  int B, H, NT;       // NT: chunk records per (sequence, head)
  int nseg, seg_len;
  int reverse;
  int whole, nch;     // state map of the whole call; chunks per sequence
  float* M_out;
  float* N_out;
};

constexpr size_t split_bytes(size_t BH, int nseg, int D) {
  return nseg > 1 ? BH * (size_t)(4 * nseg - 3) * D * D * 4 : 0;
}

// Packed sequences: sequence i is tokens [bounds[i], bounds[i + 1]) and owns
// chunk slots [cstart[i], cstart[i + 1]) of every head (both tables in the
// workspace, written by the index kernel from the caller's offsets).
struct SeqTables {
  const int* bounds;  // NULL: B equal-length sequences
  const int* cstart;
  int n_seqs;
};

struct IndexParams {
  const int* cu_seqlens;  // caller's offsets, n_seqs + 1
  int* bounds;
  int* cstart;
  int n_seqs;
  int T;
  int C;
  int* fstart;            // or NULL: first block slot per sequence for blocks of FB tokens
  int FB;
};

struct PrepParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* conv_w;        // NULL when conv_k == 0
  const void* conv_state_in;  // may be NULL
  char* ws;                 // first record
  unsigned* fb_count;       // chunks handed to the exact preparation
  unsigned* fb_list;        // their record indices
  int B, T, H, NT;
  // time slices: the records hold chunks c0 .. c0 + NT - 1 of each sequence (NT
  // record slots per (sequence, head)), and the launch covers the first nchunk of
  // them; whole sequences: c0 = 0, nchunk = NT
  int c0, nchunk;
  int conv_k;
  int l2;
  float eps;
  float scale;
  const float* A_log;    // [H]: g holds the raw gate projection (with dt_bias), or NULL
  const float* dt_bias;  // [H*D]
  int beta_logits;       // beta holds logits
  SeqTables seqs;        // packed sequences (then B = 1 and NT = chunk slots per head)
  // backward mode (all NULL otherwise): the front end's outputs in float32 --
  // y = (scale * q_hat, k_hat, v_hat) [3][B*T*H*D], gam = the chunk-local
  // cumulative log2-decay [B*T*H*D], beta [B*T*H] -- and T^T = ((I + A)^-1)^T
  // per record [C][C] in the record element type
  void* y_out;
  float* gam_out;
  float* beta_out;
  void* t_out;
};

struct StateParams {
  const char* ws;
  const float* S0;  // may be NULL; may equal S_T
  float* S_T;
  void* o;
  int B, T, H, NT;
  int c0;           // time slices: the walk takes chunks c0 .. of each sequence (0: whole)
  // output stage, applied in the walk only by the kernels built for it
  const void* o_gate;     // [B][T][H][D] or NULL
  const float* o_norm_w;  // [D] or NULL
  float o_norm_eps;
  SeqTables seqs;         // packed sequences (then B = n_seqs, NT = chunk slots per head)
  // split walk (nseg > 1; equal-length sequences, c0 = 0): one workgroup per
  // (sequence, head, segment, value block), walking chunks seg * seg_len .. of
  // its sequence from seg_start [B*H][nseg][D][D] (S0 is not read); only the
  // last segment writes S_T
  int nseg, seg_len;
  const float* seg_start;
  void* ckpt;             // backward mode: the state at each chunk start in the element type,
                          // S^T then S, [rec][2][D][D], or NULL
  // conv-state hand-over by the workgroups of value block 0, or tail_out NULL: the
  // raw q, k, v [B][T][H*D], the previous conv state (or NULL) and the new one,
  // [B][3][3][H*D].  The caller launches the walk after every read of tail_in, and
  // only with c0 = 0 (whole sequences).
  const void* tail_x[3];
  const void* tail_in;
  void* tail_out;
};

// The output stage on its own, in place on o: RMSNorm with gain and/or the
// sigmoid gate, one row of D values per (token, head).
struct OutStageParams {
  void* o;
  const void* o_gate;     // or NULL
  const float* o_norm_w;  // or NULL
  float o_norm_eps;
  long rows;
};

// ------------------------------------------------------------------ backward
// Workspace buffers of the backward pass, per record slot rec (rec_slot):
//   ckS  [rec]: S_n [D][D] (the state at the chunk start, rows = key channel) then
//        U [C][D] (the chunk's corrected values U~ - W S_n), element type
//   ckdS [rec][D][D]     dS_{n+1} (gradient of the chunk's end state), element type
//   dU   [rec][C][D]     dU_n, element type
//   dQL, dW, dKt [rec][C][D], dP [rec][C][C], dLC [rec][D]: gradients of the
//   record's quantities;  dBk, dBv [rec][C][D], dA [rec][C][C]; all in the
//   element type except dLC (float)
struct BwdWalkParams {
  const char* ws;      // forward records
  const void* dO;      // [B][T][H][D]
  const float* dS_T;   // [B][H][D][D] or NULL
  float* dS0;          // [B][H][D][D] or NULL
  void* dU;
  void* ckdS;
  int B, T, H, NT;   // B: sequences (packed: n_seqs)
  SeqTables seqs;    // packed sequences, or bounds NULL
  // split walk (nseg > 1, equal-length sequences; SplitParams): the segments'
  // reverse maps N' go to maps, the composed end gradients come from starts
  int nseg, seg_len;
  float* maps;
  float* starts;
};

struct BwdProdParams {
  const char* ws;      // forward records (W, U~)
  const void* dO;
  const void* ckS;
  const void* ckdS;
  const void* dU;
  void* dQL;
  void* dW;
  void* dKt;
  void* dP;
  float* dLC;
  int B, T, H, NT;   // B: rows of tokens (packed: 1)
  SeqTables seqs;
};

struct BwdTParams {
  const void* tT;      // T^T per record, element type
  const void* y;       // front end outputs [3][B*T*H*D], record element type
  const float* gam;
  const float* beta;
  const void* dW;
  const void* dU;
  void* dBk;
  void* dBv;
  void* dA;
  int B, T, H, NT;
  SeqTables seqs;
};

struct BwdPairParams {
  const void* y;       // front end outputs [3][B*T*H*D], record element type
  const float* gam;
  const float* beta;
  const void* dA;      // the per-record gradients in the element type (dLC float)
  const void* dP;
  const void* dQL;
  const void* dKt;
  const float* dLC;
  const void* dBk;
  const void* dBv;
  void* dy;            // [3][B*T*H*D], record element type: gradients of (scale * q_hat, k_hat, v_hat)
  float* dg;           // [B*T*H*D]
  float* dbeta_part;   // [B*T*H]: dbeta
  // chunks whose decay spans are too wide for the factored products: a count
  // (cleared before the factored kernel) and the list the per-pair kernel takes
  unsigned* ex_count;
  unsigned* ex_list;
  int B, T, H, NT;
  SeqTables seqs;
};

struct BwdFrontParams {
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;        // NULL: no convolution
  const void* conv_state_in;  // may be NULL
  const void* dy;             // [3][B*T*H*D], the I/O type
  float* dq;
  float* dk;
  float* dv;
  float* dconv_part;          // [blocks][3][H*D][4] or NULL
  float* dconv_state;         // [sequences][3][3][H*D] or NULL
  int B, T, H;
  int l2;
  float eps;
  float scale;
  // packed sequences: per sequence its first block slot (exclusive running sum
  // of its blocks of TOKB tokens); nfslots block slots per head
  SeqTables seqs;
  const int* fstart;
  int nfslots;
};

// Everything one backward launch sequence needs (the forward part is launched
// separately, in backward mode).
struct BwdLaunch {
  BwdWalkParams walk;
  BwdProdParams prod;
  BwdTParams tside;
  BwdPairParams pair;
  BwdFrontParams front;
  float* dbeta;    // [B*T*H]
  float* dconv_w;  // [3][H*D][4] or NULL
};

// Backward of the output stage (RMSNorm with gain w, then the sigmoid gate), per
// (token, head) row of D values.
struct BwdOutParams {
  const void* x;    // [rows][D] the mixer's output before the stage (I/O type)
  const void* z;    // [rows][D] gate pre-activation (I/O type) or NULL
  const void* dy;   // [rows][D] gradient of the stage's output (I/O type)
  const float* w;   // [D] gain or NULL (no norm)
  float eps;
  void* dx;         // [rows][D] gradient of x (I/O type)
  float* dz;        // [rows][D] gradient of z, or NULL
  float* dw_part;   // [groups][D] partial sums of dw (with the norm)
  long rows;        // (token, head) rows
  int H;
  SeqTables seqs;   // packed: only tokens [bounds[0], bounds[n_seqs]) count
};

// Backward of the activations from raw projections, per token and head.
struct BwdActParams {
  const void* f;          // [tokens][H][D] raw gate projection (I/O type), or NULL
  const float* A_log;     // [H]
  const float* dt_bias;   // [H*D]
  float* dg;              // [tokens][H][D] in: gradient of the decay; out: of f
  float* ddt_part;        // [groups][H*D]
  float* dA_part;         // [groups][H]
  const float* beta;      // [tokens][H] activated beta, or NULL (no logits)
  float* dbeta;           // [tokens][H] in: gradient of beta; out: of the logits
  long tokens;
  int H;
  SeqTables seqs;         // packed: only tokens [bounds[0], bounds[n_seqs]) count
};

// Most workgroups of the output-stage backward (and 1/8 of that per head for the
// activations'); their partial sums are added in a fixed order.
constexpr int kBwdStageGroups = 1024;

struct ConvNormParams {
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* conv_state_in;
  void* q_out;
  void* k_out;
  void* v_out;
  int B, T, H;
  int l2;
  float eps;
};

struct TailParams {
  const void* x[3];           // q, k, v raw inputs [B][T][H*D]
  const void* conv_state_in;  // may be NULL
  void* conv_state_out;
  int B, T, HD;
  const int* bounds;          // packed sequences: B = n_seqs, token bounds; else NULL
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* conv_w;  // NULL when conv_k == 0
  void* conv_state;
  float* S;
  void* o;
  int B, H;
  int conv_k;
  int l2;
  float eps;
  float scale;
  const float* A_log;     // as in PrepParams
  const float* dt_bias;
  int beta_logits;
  const void* o_gate;     // [B][H][D] or NULL
  const float* o_norm_w;  // [D] or NULL
  float o_norm_eps;
};

}  // namespace kda
