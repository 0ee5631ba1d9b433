// Host side of libkda: argument validation (host-only, no HIP calls), workspace
// sizing and the launch sequence on the caller's stream.  See include/kda.h.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <utility>

#include "kda_launch.h"
#include "kda_layout.h"

namespace {

using kda::record_layout;

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Span span(const void* p, size_t bytes) {
  Span s;
  if (p != nullptr && bytes > 0) {
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + bytes;
  }
  return s;
}
bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }
bool same_or_disjoint(Span a, Span b) { return (a.lo == b.lo && a.hi == b.hi) || !overlaps(a, b); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_d(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }
bool supported_chunk(int C) { return C == 16 || C == 32 || C == 64; }
size_t esize(int io) { return io == KDA_FP32 ? 4 : 2; }

// a * b * c * d without overflow past 2^62; returns false on overflow.
bool mul_ok(size_t& out, std::initializer_list<size_t> xs) {
  size_t acc = 1;
  for (size_t x : xs) {
    if (x != 0 && acc > (size_t(1) << 62) / x) return false;
    acc *= x;
  }
  out = acc;
  return true;
}

kda_status hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

struct PrefillSizes {
  size_t x;      // bytes of one [B][T][H][D] tensor
  size_t bta;    // bytes of beta
  size_t state;  // bytes of S0 / S_T
  size_t cw;     // bytes of conv_w
  size_t cst;    // bytes of a conv state
  size_t cu;     // bytes of cu_seqlens
  int NS;        // sequences: B, or n_seqs when packed
  int NT;        // chunk slots per (sequence, head), or per head when packed
};

bool packed(const kda_prefill_args* a) { return a->cu_seqlens != nullptr; }

kda_status prefill_sizes(const kda_prefill_args* a, PrefillSizes& s) {
  const size_t es = esize(a->io);
  s.NS = packed(a) ? a->n_seqs : a->B;
  size_t tok;
  if (!mul_ok(tok, {(size_t)a->B, (size_t)a->T})) return KDA_ERR_SHAPE;
  if (!mul_ok(s.x, {tok, (size_t)a->H, (size_t)a->D, es})) return KDA_ERR_SHAPE;
  if (!mul_ok(s.bta, {tok, (size_t)a->H, es})) return KDA_ERR_SHAPE;
  if (!mul_ok(s.state, {(size_t)s.NS, (size_t)a->H, (size_t)a->D, (size_t)a->D, 4})) return KDA_ERR_SHAPE;
  const size_t ck = a->conv_k > 0 ? (size_t)a->conv_k : 0;
  if (!mul_ok(s.cw, {3, (size_t)a->H, (size_t)a->D, ck, 4})) return KDA_ERR_SHAPE;
  if (!mul_ok(s.cst, {(size_t)s.NS, 3, ck > 0 ? ck - 1 : 0, (size_t)a->H, (size_t)a->D, es}))
    return KDA_ERR_SHAPE;
  s.cu = packed(a) ? ((size_t)a->n_seqs + 1) * 4 : 0;
  const long nt = a->chunk > 0 ? ((long)a->T + a->chunk - 1) / a->chunk : 0;
  // packed: every sequence wastes at most one partly filled chunk
  const long slots = packed(a) ? nt + a->n_seqs : nt;
  if (slots > 0x7fffffffL) return KDA_ERR_SHAPE;
  s.NT = (int)slots;
  // one workgroup per (b, h, chunk) and per state walk must fit a 1-D grid
  size_t wgs;
  if (!mul_ok(wgs, {(size_t)a->B, (size_t)a->H, (size_t)(s.NT > 0 ? s.NT : 1)}) ||
      wgs > 0x7fffffffu || (size_t)s.NS * a->H * 4 > 0x7fffffffu)
    return KDA_ERR_SHAPE;
  return KDA_OK;
}


// Value columns per state-walk workgroup and its thread count.  Every workgroup
// streams the chunk's W, Q Lambda, Ktil^T and P whatever its value block, so
// wider blocks read less per column; with bf16 at D = 128, 64 columns on 512
// threads measured fastest at B * H = 96 and 384.  Narrower blocks give more
// parallel walks elsewhere.
//
// With the output stage (gn) the walk applies it itself when one workgroup holds
// all D value columns (D <= 64: fused); at D = 128 o is finished by a separate
// in-place pass.  (A whole-row walk for bf16 at D = 128, 1024 threads, measured
// slower than the 64-column walk plus that pass at B * H = 96 and 384.)
struct StateCfg {
  int vb, threads;
  bool fused;
};
StateCfg state_config(int B, int H, int D, bool fp32, bool gn) {
  if (D < 64) return {D, 256, gn};
  if (gn && D == 64) return {64, 256, true};
  if (D == 128 && !fp32) return {64, 512, false};
  const long walks64 = (long)B * H * (D / 64);
  return {walks64 < 240 ? 32 : 64, 256, false};
}

// Split state walk (kda_split.hip): segments per (sequence, head) and their
// length in chunks.  Only whole-sequence walks of B equal-length sequences
// split (not time slices, packed sequences or a walk that applies the output
// stage itself); the backward's walks, forward and reverse, split as the
// forward it runs does.  Splitting adds the segment
// maps (the N and M walks of every segment but the last, about as many products
// again as the plain walk's) and a short composition in exchange for a chain of
// seg_len instead of all chunk steps, which pays while the walks leave CUs idle:
// at most kSplitWalks workgroups in the split walk, segments of at least
// kMinSegChunks chunks, and at most kMaxSegments segments (the composition is a
// chain of nseg - 2 D x D products).
struct SplitPlan {
  int nseg = 1, seg_len = 0;
};
constexpr long kSplitWalks = 256;
constexpr int kMinSegChunks = 16;
constexpr long kMaxSegments = 32;

SplitPlan split_plan(const kda_prefill_args* a) {
  SplitPlan sp;
  if (packed(a) || a->T <= 0 || a->chunk <= 0) return sp;
  const bool gn = a->o_norm_w != nullptr || a->o_gate != nullptr;
  const StateCfg cfg = state_config(a->B, a->H, a->D, a->io == KDA_FP32, gn);
  if (cfg.fused) return sp;
  const long walks = (long)a->B * a->H * (a->D / cfg.vb);
  const long nch = ((long)a->T + a->chunk - 1) / a->chunk;
  long P = kSplitWalks / walks;
  if (nch / kMinSegChunks < P) P = nch / kMinSegChunks;
  if (kMaxSegments < P) P = kMaxSegments;
  if (P < 2) return sp;
  sp.seg_len = (int)((nch + P - 1) / P);
  sp.nseg = (int)((nch + sp.seg_len - 1) / sp.seg_len);
  if (sp.nseg < 2) sp = SplitPlan{};
  return sp;
}

// The state map of a whole call (kda_prefill_state_map) cuts the walks as the
// split walk would, but into at least one segment, and maps every segment.
SplitPlan map_plan(const kda_prefill_args* a) {
  SplitPlan sp;
  if (a->T <= 0 || a->chunk <= 0) return sp;
  const StateCfg cfg = state_config(a->B, a->H, a->D, a->io == KDA_FP32, false);
  const long walks = (long)a->B * a->H * (a->D / cfg.vb);
  const long nch = ((long)a->T + a->chunk - 1) / a->chunk;
  long P = kSplitWalks / walks;
  if (nch / kMinSegChunks < P) P = nch / kMinSegChunks;
  if (kMaxSegments < P) P = kMaxSegments;
  if (P < 1) P = 1;
  sp.seg_len = (int)((nch + P - 1) / P);
  sp.nseg = (int)((nch + sp.seg_len - 1) / sp.seg_len);
  return sp;
}

kda::WorkspaceLayout ws_layout(const kda_prefill_args* a) {
  PrefillSizes s;
  prefill_sizes(a, s);
  const SplitPlan sp = split_plan(a);
  return kda::workspace_layout((size_t)a->B * a->H * s.NT, a->chunk, a->D, esize(a->io),
                               packed(a) ? (size_t)a->n_seqs : 0,
                               kda::split_bytes((size_t)a->B * a->H, sp.nseg, a->D));
}

constexpr uint32_t kKnownFlags = KDA_FLAG_L2NORM_QK | KDA_FLAG_BETA_LOGITS;

// Checks shared by prefill and decode for the optional stages' pointers and
// scalars (their overlaps are checked with the other buffers).
kda_status validate_stages(const float* A_log, const float* dt_bias, const float* o_norm_w,
                           float o_norm_eps, const void* o_gate) {
  if ((A_log == nullptr) != (dt_bias == nullptr)) return KDA_ERR_NULL;
  if (o_norm_w != nullptr && (!std::isfinite(o_norm_eps) || o_norm_eps < 0.f)) return KDA_ERR_VALUE;
  for (const void* p : {(const void*)A_log, (const void*)dt_bias, (const void*)o_norm_w, o_gate})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid or overflowing size";
    case KDA_ERR_DTYPE: return "invalid dtype";
    case KDA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case KDA_ERR_ALIAS: return "output overlaps an input";
    case KDA_ERR_UNSUPPORTED: return "unsupported mode";
    case KDA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_VALUE: return "scalar argument out of range";
    case KDA_ERR_SCRATCH: return "request needs more than the static scratch buffer";
  }
  return "unknown status";
}

kda_status kda_validate_prefill(const kda_prefill_args* a) {
  if (a == nullptr) return KDA_ERR_NULL;
  if (a->io != KDA_BF16 && a->io != KDA_FP32) return KDA_ERR_DTYPE;
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->D < 1 || a->chunk < 1 || a->conv_k < 0)
    return KDA_ERR_SHAPE;
  if (!supported_d(a->D) || !supported_chunk(a->chunk) || (a->conv_k != 0 && a->conv_k != 4))
    return KDA_ERR_UNSUPPORTED;
  if (a->io == KDA_FP32 && a->D == 128 && a->chunk == 64) return KDA_ERR_UNSUPPORTED;
  if ((a->flags & ~kKnownFlags) != 0) return KDA_ERR_VALUE;
  if (!std::isfinite(a->l2_eps) || a->l2_eps < 0.f || !std::isfinite(a->scale)) return KDA_ERR_VALUE;
  PrefillSizes s;
  if (kda_status e = prefill_sizes(a, s); e != KDA_OK) return e;
  if (kda_status e = validate_stages(a->A_log, a->dt_bias, a->o_norm_w, a->o_norm_eps, a->o_gate);
      e != KDA_OK)
    return e;
  if (packed(a) ? (a->B != 1 || a->n_seqs < 1) : a->n_seqs != 0) return KDA_ERR_SHAPE;
  const bool need_x = a->T > 0;
  if (need_x && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o)) return KDA_ERR_NULL;
  if (!a->S_T) return KDA_ERR_NULL;
  if (a->conv_k > 0 && !a->conv_w) return KDA_ERR_NULL;
  if (a->conv_k == 0 && (a->conv_w || a->conv_state_in || a->conv_state_out)) return KDA_ERR_NULL;
  for (const void* p : std::initializer_list<const void*>{a->q, a->k, a->v, a->g, a->beta, (const void*)a->conv_w, a->conv_state_in,
                        (const void*)a->S0, a->o, (const void*)a->S_T, (const void*)a->conv_state_out,
                        (const void*)a->cu_seqlens})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const Span q = span(a->q, s.x), k = span(a->k, s.x), v = span(a->v, s.x), g = span(a->g, s.x);
  const Span bt = span(a->beta, s.bta), cw = span(a->conv_w, s.cw);
  const Span ci = span(a->conv_state_in, s.cst), co = span(a->conv_state_out, s.cst);
  const Span s0 = span(a->S0, s.state), st = span(a->S_T, s.state), o = span(a->o, s.x);
  const Span al = span(a->A_log, (size_t)a->H * 4), db = span(a->dt_bias, (size_t)a->H * a->D * 4);
  const Span nw = span(a->o_norm_w, (size_t)a->D * 4), og = span(a->o_gate, s.x);
  const Span cu = span(a->cu_seqlens, s.cu);
  for (Span in : {q, k, v, g, bt, cw, ci, s0, st, co, al, db, nw, og, cu})
    if (overlaps(o, in)) return KDA_ERR_ALIAS;
  for (Span in : {q, k, v, g, bt, cw, ci, co, al, db, nw, og, cu})
    if (overlaps(st, in)) return KDA_ERR_ALIAS;
  if (!same_or_disjoint(st, s0)) return KDA_ERR_ALIAS;
  for (Span in : {q, k, v, g, bt, cw, s0, al, db, nw, og, cu})
    if (overlaps(co, in)) return KDA_ERR_ALIAS;
  if (!same_or_disjoint(co, ci)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

size_t kda_prefill_workspace_bytes(const kda_prefill_args* a) {
  if (kda_validate_prefill(a) != KDA_OK) return 0;
  if (a->T == 0) return 0;
  PrefillSizes s;
  prefill_sizes(a, s);
  size_t n;
  const size_t rec = record_layout(a->chunk, a->D, esize(a->io)).bytes;
  if (!mul_ok(n, {(size_t)a->B, (size_t)a->H, (size_t)s.NT, rec})) return 0;
  return ws_layout(a).bytes;
}

// The workspace of a call: 256-byte aligned, at least `need` bytes (the
// prefill's by default), and clear of every buffer of the call.
static kda_status check_workspace(const kda_prefill_args* a, void* ws, size_t ws_bytes,
                                  size_t need = 0) {
  if (need == 0) need = kda_prefill_workspace_bytes(a);
  if (need == 0) return KDA_OK;
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < need)
    return KDA_ERR_WORKSPACE;
  PrefillSizes s;
  prefill_sizes(a, s);
  const Span w = span(ws, need);
  for (Span x : {span(a->q, s.x), span(a->k, s.x), span(a->v, s.x), span(a->g, s.x),
                 span(a->beta, s.bta), span(a->conv_w, s.cw), span(a->conv_state_in, s.cst),
                 span(a->S0, s.state), span(a->o, s.x), span(a->S_T, s.state),
                 span(a->conv_state_out, s.cst), span(a->A_log, (size_t)a->H * 4),
                 span(a->dt_bias, (size_t)a->H * a->D * 4), span(a->o_norm_w, (size_t)a->D * 4),
                 span(a->o_gate, s.x), span(a->cu_seqlens, s.cu)})
    if (overlaps(w, x)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

// The packed-sequence tables in the workspace (written by the first stage).
static kda::SeqTables seq_tables(const kda_prefill_args* a, void* ws) {
  kda::SeqTables t{};
  if (!packed(a) || a->T == 0) return t;
  int* bounds = reinterpret_cast<int*>(static_cast<char*>(ws) + ws_layout(a).seq);
  t.bounds = bounds;
  t.cstart = bounds + a->n_seqs + 1;
  t.n_seqs = a->n_seqs;
  return t;
}

// Extra outputs of the forward stages when they run for the backward pass.
struct BwdFwdOut {
  void* y;
  float* gam;
  float* beta;
  void* tT;  // record element type
  void* ckS;
};

// A time slice of B equal-length sequences: chunks c0 .. c0 + cnt - 1 of every
// sequence, whose records take cap slots per (sequence, head) of a workspace laid
// out for B * H * cap records.  cap = 0: whole sequences.
struct Slice {
  int c0 = 0, cnt = 0, cap = 0;
};

// fuse_tail: the state walk (T > 0) also writes the conv-state hand-over, and
// the hand-over stage does nothing then.  A slice (sl != NULL) prepares or walks
// only its chunks; its walk starts from S0 when c0 = 0 and from S_T (the previous
// slice's end state) otherwise.
static kda_status run_stage(const kda_prefill_args* a, void* ws, int stage, hipStream_t st,
                            const BwdFwdOut* bo = nullptr, bool fuse_tail = false,
                            const Slice* sl = nullptr) {
  const bool fp32 = a->io == KDA_FP32;
  PrefillSizes sz;
  prefill_sizes(a, sz);
  const int NT = sl != nullptr ? sl->cap : sz.NT;
  const kda::SeqTables seqs = sl != nullptr ? kda::SeqTables{} : seq_tables(a, ws);
  const kda::WorkspaceLayout wl =
      sl != nullptr ? kda::workspace_layout((size_t)a->B * a->H * sl->cap, a->chunk, a->D, esize(a->io))
                    : ws_layout(a);
  switch (stage) {
    case KDA_STAGE_PREP: {
      if (a->T == 0) return KDA_OK;
      if (packed(a)) {
        kda::IndexParams ip{};
        ip.cu_seqlens = a->cu_seqlens;
        ip.bounds = const_cast<int*>(seqs.bounds);
        ip.cstart = const_cast<int*>(seqs.cstart);
        ip.n_seqs = a->n_seqs;
        ip.T = a->T;
        ip.C = a->chunk;
        if (kda_status e = hip_status(kda::launch_seq_index(ip, st)); e != KDA_OK) return e;
      }
      kda::PrepParams p{};
      p.q = a->q; p.k = a->k; p.v = a->v; p.g = a->g; p.beta = a->beta;
      p.conv_w = a->conv_k > 0 ? a->conv_w : nullptr;
      p.conv_state_in = a->conv_k > 0 ? a->conv_state_in : nullptr;
      p.ws = static_cast<char*>(ws) + wl.records;
      p.fb_count = static_cast<unsigned*>(ws);
      p.fb_list = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + wl.list);
      p.B = a->B; p.T = a->T; p.H = a->H; p.NT = NT;
      p.c0 = sl != nullptr ? sl->c0 : 0;
      p.nchunk = sl != nullptr ? sl->cnt : NT;
      p.conv_k = a->conv_k;
      p.l2 = (a->flags & KDA_FLAG_L2NORM_QK) ? 1 : 0;
      p.eps = a->l2_eps;
      p.scale = a->scale;
      p.A_log = a->A_log;
      p.dt_bias = a->dt_bias;
      p.beta_logits = (a->flags & KDA_FLAG_BETA_LOGITS) ? 1 : 0;
      p.seqs = seqs;
      if (bo != nullptr) {
        p.y_out = bo->y;
        p.gam_out = bo->gam;
        p.beta_out = bo->beta;
        p.t_out = bo->tT;
      }
      return hip_status(kda::launch_prep(p, a->D, a->chunk, fp32, st));
    }
    case KDA_STAGE_STATE: {
      if (a->T == 0) {
        if (a->S_T == a->S0) return KDA_OK;
        const size_t n = (size_t)sz.NS * a->H * a->D * a->D;
        return hip_status(kda::launch_copy_state(a->S0, a->S_T, n, st));
      }
      const bool gn = a->o_norm_w != nullptr || a->o_gate != nullptr;
      const StateCfg cfg = state_config(sz.NS, a->H, a->D, fp32, gn);
      kda::StateParams p{};
      p.ws = static_cast<const char*>(ws) + wl.records;
      p.S0 = sl != nullptr && sl->c0 > 0 ? a->S_T : a->S0;
      p.S_T = a->S_T; p.o = a->o;
      p.B = sz.NS; p.T = a->T; p.H = a->H; p.NT = NT;
      p.c0 = sl != nullptr ? sl->c0 : 0;
      p.seqs = seqs;
      p.o_gate = a->o_gate;
      p.o_norm_w = a->o_norm_w;
      p.o_norm_eps = a->o_norm_eps;
      p.ckpt = bo != nullptr ? bo->ckS : nullptr;
      const SplitPlan sp = sl == nullptr ? split_plan(a) : SplitPlan{};
      if (sp.nseg > 1) {
        kda::SplitParams q{};
        q.ws = p.ws;
        q.S0 = a->S0;
        q.maps = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.split);
        q.starts = q.maps + (size_t)a->B * a->H * (sp.nseg - 1) * 3 * a->D * a->D;
        q.B = a->B; q.H = a->H; q.NT = NT;
        q.nseg = sp.nseg; q.seg_len = sp.seg_len;
        if (kda_status e = hip_status(kda::launch_split_maps(q, a->D, a->chunk, fp32, cfg.vb,
                                                             cfg.threads, st));
            e != KDA_OK)
          return e;
        if (kda_status e = hip_status(kda::launch_split_combine(q, a->D, st)); e != KDA_OK) return e;
        p.nseg = sp.nseg;
        p.seg_len = sp.seg_len;
        p.seg_start = q.starts;
      }
      if (fuse_tail && sl == nullptr && a->conv_k > 0 && a->conv_state_out != nullptr) {
        p.tail_x[0] = a->q; p.tail_x[1] = a->k; p.tail_x[2] = a->v;
        p.tail_in = a->conv_state_in;
        p.tail_out = a->conv_state_out;
      }
      return hip_status(kda::launch_state(p, a->D, a->chunk, fp32, cfg.vb, cfg.threads, cfg.fused,
                                          st));
    }
    case KDA_STAGE_OUTPUT: {
      const bool gn = a->o_norm_w != nullptr || a->o_gate != nullptr;
      if (a->T == 0 || !gn || state_config(sz.NS, a->H, a->D, fp32, gn).fused) return KDA_OK;
      kda::OutStageParams q{};
      q.o = a->o;
      q.o_gate = a->o_gate;
      q.o_norm_w = a->o_norm_w;
      q.o_norm_eps = a->o_norm_eps;
      q.rows = (long)a->B * a->T * a->H;
      return hip_status(kda::launch_out_stage(q, a->D, fp32, st));
    }
    case KDA_STAGE_CONV_TAIL: {
      if (a->conv_k == 0 || a->conv_state_out == nullptr || (fuse_tail && sl == nullptr && a->T > 0))
        return KDA_OK;
      kda::TailParams p{};
      p.x[0] = a->q; p.x[1] = a->k; p.x[2] = a->v;
      p.conv_state_in = a->conv_state_in;
      p.conv_state_out = a->conv_state_out;
      p.B = sz.NS; p.T = a->T; p.HD = a->H * a->D;
      p.bounds = seqs.bounds;  // NULL unless packed with T > 0 (T = 0: every sequence is empty)
      return hip_status(kda::launch_conv_tail(p, fp32, st));
    }
  }
  return KDA_ERR_VALUE;
}

// Largest number of chunk slots per (sequence, head) whose workspace fits `bytes`
// (at most the sequence's chunk count), or 0 when not even one fits.
static int slice_capacity(const kda_prefill_args* a, size_t bytes) {
  const int nt = (a->T + a->chunk - 1) / a->chunk;
  const size_t bh = (size_t)a->B * a->H;
  int lo = 0, hi = nt;  // workspace_layout grows with the slot count
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (kda::workspace_layout(bh * mid, a->chunk, a->D, esize(a->io)).bytes <= bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // extern "C"

namespace kda {

// The whole forward in a caller-sized workspace (validated arguments): as
// kda_prefill when its workspace fits `bytes`; otherwise B equal-length
// sequences are run in time slices (preparation and walk of as many chunks per
// (sequence, head) as fit, the state carried from one slice to the next in S_T),
// then the conv hand-over and the separate output pass over whole sequences.
kda_status prefill_in_workspace(const kda_prefill_args* a, void* ws, size_t bytes, hipStream_t st) {
  if (a->T > 0 && ws_layout(a).bytes > bytes) {
    if (packed(a)) return KDA_ERR_SCRATCH;
    const int cap = slice_capacity(a, bytes);
    if (cap < 1) return KDA_ERR_SCRATCH;
    const int nt = (a->T + a->chunk - 1) / a->chunk;
    for (int c0 = 0; c0 < nt; c0 += cap) {
      const Slice sl{c0, nt - c0 < cap ? nt - c0 : cap, cap};
      if (kda_status e = run_stage(a, ws, KDA_STAGE_PREP, st, nullptr, false, &sl); e != KDA_OK)
        return e;
      if (kda_status e = run_stage(a, ws, KDA_STAGE_STATE, st, nullptr, false, &sl); e != KDA_OK)
        return e;
    }
    if (kda_status e = run_stage(a, ws, KDA_STAGE_CONV_TAIL, st); e != KDA_OK) return e;
    return run_stage(a, ws, KDA_STAGE_OUTPUT, st);
  }
  for (int stage = KDA_STAGE_PREP; stage <= KDA_STAGE_OUTPUT; ++stage)
    if (kda_status e = run_stage(a, ws, stage, st, nullptr, true); e != KDA_OK) return e;
  return KDA_OK;
}

}  // namespace kda

extern "C" {

kda_status kda_prefill_stage(const kda_prefill_args* a, void* ws, size_t ws_bytes, int stage,
                             void* stream) {
  if (kda_status e = kda_validate_prefill(a); e != KDA_OK) return e;
  if (stage < KDA_STAGE_PREP || stage > KDA_STAGE_STATE_TAIL) return KDA_ERR_VALUE;
  if (kda_status e = check_workspace(a, ws, ws_bytes); e != KDA_OK) return e;
  if (stage == KDA_STAGE_STATE_TAIL)
    return run_stage(a, ws, KDA_STAGE_STATE, static_cast<hipStream_t>(stream), nullptr, true);
  return run_stage(a, ws, stage, static_cast<hipStream_t>(stream));
}

size_t kda_prefill_state_map_workspace_bytes(const kda_prefill_args* a) {
  if (kda_validate_prefill(a) != KDA_OK || packed(a) || a->T == 0) return 0;
  const kda::WorkspaceLayout wl = ws_layout(a);
  const SplitPlan sp = map_plan(a);
  const size_t maps = (size_t)a->B * a->H * sp.nseg * 3 * a->D * a->D * 4;
  return wl.split + maps > wl.bytes ? wl.split + maps : wl.bytes;
}

kda_status kda_prefill_state_map(const kda_prefill_args* a, void* ws, size_t ws_bytes, float* M,
                                 float* N, void* stream) {
  if (kda_status e = kda_validate_prefill(a); e != KDA_OK) return e;
  if (packed(a)) return KDA_ERR_UNSUPPORTED;
  if (M == nullptr || N == nullptr) return KDA_ERR_NULL;
  if (!aligned16(M) || !aligned16(N)) return KDA_ERR_ALIGN;
  PrefillSizes sz;
  prefill_sizes(a, sz);
  const Span m = span(M, sz.state), n = span(N, sz.state);
  if (overlaps(m, n)) return KDA_ERR_ALIAS;
  for (Span x : {span(a->q, sz.x), span(a->k, sz.x), span(a->v, sz.x), span(a->g, sz.x),
                 span(a->beta, sz.bta), span(a->conv_w, sz.cw), span(a->conv_state_in, sz.cst),
                 span(a->S0, sz.state), span(a->o, sz.x), span(a->S_T, sz.state),
                 span(a->conv_state_out, sz.cst), span(a->A_log, (size_t)a->H * 4),
                 span(a->dt_bias, (size_t)a->H * a->D * 4), span(a->o_norm_w, (size_t)a->D * 4),
                 span(a->o_gate, sz.x)})
    if (overlaps(m, x) || overlaps(n, x)) return KDA_ERR_ALIAS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a->T == 0)
    return hip_status(kda::launch_state_map_identity(M, N, (size_t)a->B * a->H * a->D * a->D, a->D, st));
  const size_t need = kda_prefill_state_map_workspace_bytes(a);
  if (kda_status e = check_workspace(a, ws, ws_bytes, need); e != KDA_OK) return e;
  const Span w = span(ws, need);
  if (overlaps(w, m) || overlaps(w, n)) return KDA_ERR_ALIAS;
  const kda::WorkspaceLayout wl = ws_layout(a);
  const SplitPlan sp = map_plan(a);
  const StateCfg cfg = state_config(a->B, a->H, a->D, a->io == KDA_FP32, false);
  kda::SplitParams q{};
  q.ws = static_cast<const char*>(ws) + wl.records;
  q.maps = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.split);
  q.B = a->B; q.H = a->H; q.NT = sz.NT;
  q.nseg = sp.nseg; q.seg_len = sp.seg_len;
  q.whole = 1;
  q.nch = (a->T + a->chunk - 1) / a->chunk;
  q.M_out = M;
  q.N_out = N;
  return hip_status(kda::launch_state_map(q, a->D, a->chunk, a->io == KDA_FP32, cfg.vb, cfg.threads, st));
}

int kda_prefill_walk_segments(const kda_prefill_args* a) {
  if (kda_validate_prefill(a) != KDA_OK) return 0;
  return split_plan(a).nseg;
}

kda_status kda_prefill(const kda_prefill_args* a, void* ws, size_t ws_bytes, void* stream) {
  if (kda_status e = kda_validate_prefill(a); e != KDA_OK) return e;
  if (kda_status e = check_workspace(a, ws, ws_bytes); e != KDA_OK) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // stages 0, 4, 3 (stage 4 is the walk with the hand-over; the hand-over stage is
  // then empty, and so is the state stage when T = 0 leaves the hand-over to it)
  for (int stage = KDA_STAGE_PREP; stage <= KDA_STAGE_OUTPUT; ++stage)
    if (kda_status e = run_stage(a, ws, stage, st, nullptr, true); e != KDA_OK) return e;
  return KDA_OK;
}

// ------------------------------------------------------------------ conv_norm
kda_status kda_validate_conv_norm(const kda_conv_norm_args* a) {
  if (a == nullptr) return KDA_ERR_NULL;
  if (a->io != KDA_BF16 && a->io != KDA_FP32) return KDA_ERR_DTYPE;
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->D < 1 || a->conv_k < 0) return KDA_ERR_SHAPE;
  if (!supported_d(a->D) || a->conv_k != 4) return KDA_ERR_UNSUPPORTED;
  if ((a->flags & ~KDA_FLAG_L2NORM_QK) != 0) return KDA_ERR_VALUE;
  if (!std::isfinite(a->l2_eps) || a->l2_eps < 0.f) return KDA_ERR_VALUE;
  const size_t es = esize(a->io);
  size_t x, cw, cst;
  if (!mul_ok(x, {(size_t)a->B, (size_t)a->T, (size_t)a->H, (size_t)a->D, es}) ||
      !mul_ok(cw, {3, (size_t)a->H, (size_t)a->D, 4, 4}) ||
      !mul_ok(cst, {(size_t)a->B, 3, 3, (size_t)a->H, (size_t)a->D, es}))
    return KDA_ERR_SHAPE;
  if ((size_t)a->B * a->H * ((a->T + 63) / 64 + 1) > 0x7fffffffu) return KDA_ERR_SHAPE;
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->q_out || !a->k_out || !a->v_out))
    return KDA_ERR_NULL;
  if (!a->conv_w) return KDA_ERR_NULL;
  for (const void* p : std::initializer_list<const void*>{a->q, a->k, a->v, (const void*)a->conv_w, a->conv_state_in, a->q_out,
                        a->k_out, a->v_out, a->conv_state_out})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const Span q = span(a->q, x), k = span(a->k, x), v = span(a->v, x), w = span(a->conv_w, cw);
  const Span ci = span(a->conv_state_in, cst), co = span(a->conv_state_out, cst);
  const Span oq = span(a->q_out, x), ok = span(a->k_out, x), ov = span(a->v_out, x);
  for (Span out : {oq, ok, ov})
    for (Span in : {q, k, v, w, ci, co})
      if (overlaps(out, in)) return KDA_ERR_ALIAS;
  if (overlaps(oq, ok) || overlaps(oq, ov) || overlaps(ok, ov)) return KDA_ERR_ALIAS;
  for (Span in : {q, k, v, w})
    if (overlaps(co, in)) return KDA_ERR_ALIAS;
  if (!same_or_disjoint(co, ci)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status kda_conv_norm(const kda_conv_norm_args* a, void* stream) {
  if (kda_status e = kda_validate_conv_norm(a); e != KDA_OK) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fp32 = a->io == KDA_FP32;
  if (a->T > 0) {
    kda::ConvNormParams p{};
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.conv_w = a->conv_w;
    p.conv_state_in = a->conv_state_in;
    p.q_out = a->q_out; p.k_out = a->k_out; p.v_out = a->v_out;
    p.B = a->B; p.T = a->T; p.H = a->H;
    p.l2 = (a->flags & KDA_FLAG_L2NORM_QK) ? 1 : 0;
    p.eps = a->l2_eps;
    if (kda_status e = hip_status(kda::launch_conv_norm(p, a->D, fp32, st)); e != KDA_OK) return e;
  }
  if (a->conv_state_out != nullptr) {
    kda::TailParams p{};
    p.x[0] = a->q; p.x[1] = a->k; p.x[2] = a->v;
    p.conv_state_in = a->conv_state_in;
    p.conv_state_out = a->conv_state_out;
    p.B = a->B; p.T = a->T; p.HD = a->H * a->D;
    return hip_status(kda::launch_conv_tail(p, fp32, st));
  }
  return KDA_OK;
}

// --------------------------------------------------------------------- decode
kda_status kda_validate_decode(const kda_decode_args* a) {
  if (a == nullptr) return KDA_ERR_NULL;
  if (a->io != KDA_BF16 && a->io != KDA_FP32) return KDA_ERR_DTYPE;
  if (a->B < 1 || a->H < 1 || a->D < 1 || a->conv_k < 0) return KDA_ERR_SHAPE;
  if (!supported_d(a->D) || (a->conv_k != 0 && a->conv_k != 4)) return KDA_ERR_UNSUPPORTED;
  if ((a->flags & ~kKnownFlags) != 0) return KDA_ERR_VALUE;
  if (!std::isfinite(a->l2_eps) || a->l2_eps < 0.f || !std::isfinite(a->scale)) return KDA_ERR_VALUE;
  if (kda_status e = validate_stages(a->A_log, a->dt_bias, a->o_norm_w, a->o_norm_eps, a->o_gate);
      e != KDA_OK)
    return e;
  const size_t es = esize(a->io);
  const size_t ck = a->conv_k > 0 ? (size_t)a->conv_k : 0;
  size_t x, bt, st, cw, cst;
  if (!mul_ok(x, {(size_t)a->B, (size_t)a->H, (size_t)a->D, es}) ||
      !mul_ok(bt, {(size_t)a->B, (size_t)a->H, es}) ||
      !mul_ok(st, {(size_t)a->B, (size_t)a->H, (size_t)a->D, (size_t)a->D, 4}) ||
      !mul_ok(cw, {3, (size_t)a->H, (size_t)a->D, ck, 4}) ||
      !mul_ok(cst, {(size_t)a->B, 3, ck > 0 ? ck - 1 : 0, (size_t)a->H, (size_t)a->D, es}))
    return KDA_ERR_SHAPE;
  if ((size_t)a->B * a->H > 0x7fffffffu) return KDA_ERR_SHAPE;
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->S || !a->o) return KDA_ERR_NULL;
  if (a->conv_k > 0 && (!a->conv_w || !a->conv_state)) return KDA_ERR_NULL;
  if (a->conv_k == 0 && (a->conv_w || a->conv_state)) return KDA_ERR_NULL;
  for (const void* p : std::initializer_list<const void*>{a->q, a->k, a->v, a->g, a->beta, (const void*)a->conv_w,
                        (const void*)a->conv_state, (const void*)a->S, a->o})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const Span q = span(a->q, x), k = span(a->k, x), v = span(a->v, x), g = span(a->g, x);
  const Span b = span(a->beta, bt), w = span(a->conv_w, cw), cs = span(a->conv_state, cst);
  const Span S = span(a->S, st), o = span(a->o, x);
  const Span al = span(a->A_log, (size_t)a->H * 4), db = span(a->dt_bias, (size_t)a->H * a->D * 4);
  const Span nw = span(a->o_norm_w, (size_t)a->D * 4), og = span(a->o_gate, x);
  for (Span in : {q, k, v, g, b, w, cs, S, al, db, nw, og})
    if (overlaps(o, in)) return KDA_ERR_ALIAS;
  for (Span in : {q, k, v, g, b, w, cs, al, db, nw, og})
    if (overlaps(S, in)) return KDA_ERR_ALIAS;
  for (Span in : {q, k, v, g, b, w, al, db, nw, og})
    if (overlaps(cs, in)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

kda_status kda_decode_step(const kda_decode_args* a, void* stream) {
  if (kda_status e = kda_validate_decode(a); e != KDA_OK) return e;
  kda::DecodeParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.g = a->g; p.beta = a->beta;
  p.conv_w = a->conv_k > 0 ? a->conv_w : nullptr;
  p.conv_state = a->conv_state;
  p.S = a->S;
  p.o = a->o;
  p.B = a->B; p.H = a->H;
  p.conv_k = a->conv_k;
  p.l2 = (a->flags & KDA_FLAG_L2NORM_QK) ? 1 : 0;
  p.eps = a->l2_eps;
  p.scale = a->scale;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.beta_logits = (a->flags & KDA_FLAG_BETA_LOGITS) ? 1 : 0;
  p.o_gate = a->o_gate;
  p.o_norm_w = a->o_norm_w;
  p.o_norm_eps = a->o_norm_eps;
  return hip_status(kda::launch_decode(p, a->D, a->io == KDA_FP32, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------- backward
}  // extern "C"

namespace {

// Workspace of the backward pass: the forward workspace, then float32 buffers
// (see kda_layout.h), each 256-byte aligned.
struct BwdLayout {
  size_t tT, y, gam, beta, ckS, ckdS, dU, dQL, dW, dKt, dP, dLC, dBk, dBv, dA, dy, dbp, dcp, pl;
  size_t dOp, dwp, ddp, dap;  // the optional stages: dO before the output stage, partial sums
  size_t fst;                 // packed: first front-end block slot per sequence [n_seqs + 1]
  size_t opre;                // saved forward with the output stage: the mixer's output
  size_t bytes;
  size_t nfront;  // front-end block slots per head (filter partials)
};

// The forward that the backward runs: the mixer without the output stage (the
// stage is differentiated and applied separately).  Its workspace layout, split
// walk included, is the base of the backward's.
kda_prefill_args forward_of_backward(const kda_prefill_args* f) {
  kda_prefill_args f0 = *f;
  f0.o_norm_w = nullptr;
  f0.o_gate = nullptr;
  return f0;
}

// saved: the workspace of kda_prefill_forward_saved / kda_prefill_backward_saved,
// which also keeps the mixer's output before the output stage.  The layout
// depends on the forward's arguments only.
BwdLayout bwd_layout(const kda_backward_args* a, bool saved = false) {
  const kda_prefill_args* f = &a->fwd;
  const kda_prefill_args f0 = forward_of_backward(f);
  BwdLayout L{};
  PrefillSizes sz;
  prefill_sizes(f, sz);
  const size_t nrec = (size_t)f->B * f->H * sz.NT;
  const size_t C = (size_t)f->chunk, D = (size_t)f->D;
  const size_t x = (size_t)f->B * f->T * f->H * D;  // elements of one [B][T][H][D] tensor
  const size_t bth = (size_t)f->B * f->T * f->H;
  size_t off = kda::round_up(ws_layout(&f0).bytes, 256);
  auto take = [&](size_t floats) {
    const size_t o = off;
    off = kda::round_up(off + floats * 4, 256);
    return o;
  };
  const size_t ef = esize(f->io) == 2 ? 2 : 1;  // element-type buffers in float units (rounded up)
  L.tT = take(nrec * C * C / ef);  // T^T in the record element type
  L.y = take(3 * x / ef);  // front end outputs in the record element type
  L.gam = take(x);
  L.beta = take(bth);
  L.ckS = take(nrec * (D * D + C * D) / ef);  // S_n [D][D] and U [C][D] per record
  L.ckdS = take(nrec * D * D / ef);
  L.dU = take(nrec * C * D / ef);
  // per-record gradients in the record element type (dLC in float)
  L.dQL = take(nrec * C * D / ef);
  L.dW = take(nrec * C * D / ef);
  L.dKt = take(nrec * C * D / ef);
  L.dP = take(nrec * C * C / ef);
  L.dLC = take(nrec * D);
  L.dBk = take(nrec * C * D / ef);
  L.dBv = take(nrec * C * D / ef);
  L.dA = take(nrec * C * C / ef);
  L.dy = take(3 * x / ef);  // record element type
  L.dbp = take(bth);
  // front-end block slots: per (sequence, block of the sequence) for packed
  // batches, ceil(T / TOKB) + n_seqs of them (a sequence wastes at most one block)
  L.nfront = packed(f) ? kda::bwd_front_blocks(f->T, f->D) + (size_t)f->n_seqs
                       : (size_t)f->B * kda::bwd_front_blocks(f->T, f->D);
  L.dcp = take(f->conv_k > 0 ? L.nfront * 3 * f->H * D * 4 : 0);
  L.fst = take(packed(f) ? (size_t)f->n_seqs + 1 : 0);
  L.pl = take(64 + nrec);  // count (256-byte header), then the list of records
  const bool gn = f->o_norm_w != nullptr || f->o_gate != nullptr;
  L.dOp = take(gn ? x / ef : 0);  // gradient of the mixer's output (before the stage), I/O type
  L.dwp = take(f->o_norm_w != nullptr ? (size_t)kda::bwd_out_groups((long)bth, f->D) * D : 0);
  const size_t nact = f->A_log != nullptr ? (size_t)kda::bwd_act_groups((long)f->B * f->T, f->D) : 0;
  L.ddp = take(nact * f->H * D);
  L.dap = take(nact * f->H);
  L.opre = take(saved && gn ? x / ef : 0);  // I/O type
  L.bytes = off;
  return L;
}

// Every buffer of a backward call with its byte size: 17 inputs (and forward
// outputs), 12 gradient outputs.
constexpr int kBwdIns = 17, kBwdOuts = 12;
void bwd_spans(const kda_backward_args* a, Span (&ins)[kBwdIns], Span (&outs)[kBwdOuts]) {
  const kda_prefill_args* f = &a->fwd;
  PrefillSizes s;
  prefill_sizes(f, s);
  const size_t g = (size_t)f->B * f->T * f->H * f->D * 4, gb = (size_t)f->B * f->T * f->H * 4;
  const size_t ck = f->conv_k > 0 ? (size_t)f->conv_k - 1 : 0;
  const size_t dcs = (size_t)s.NS * 3 * ck * f->H * f->D * 4;
  const size_t H4 = (size_t)f->H * 4, HD4 = (size_t)f->H * f->D * 4, D4 = (size_t)f->D * 4;
  const Span i[kBwdIns] = {span(f->q, s.x), span(f->k, s.x), span(f->v, s.x), span(f->g, s.x),
                           span(f->beta, s.bta), span(f->conv_w, s.cw), span(f->conv_state_in, s.cst),
                           span(f->S0, s.state), span(f->o, s.x), span(f->S_T, s.state),
                           span(f->conv_state_out, s.cst), span(a->dO, s.x), span(a->dS_T, s.state),
                           span(f->A_log, H4), span(f->dt_bias, HD4), span(f->o_norm_w, D4),
                           span(f->o_gate, s.x)};
  const Span o[kBwdOuts] = {span(a->dq, g), span(a->dk, g), span(a->dv, g), span(a->dg, g),
                            span(a->dbeta, gb), span(a->dS0, s.state), span(a->dconv_w, s.cw),
                            span(a->dconv_state, dcs), span(a->dA_log, H4), span(a->ddt_bias, HD4),
                            span(a->do_norm_w, D4), span(a->do_gate, g)};
  for (int k = 0; k < kBwdIns; ++k) ins[k] = i[k];
  for (int k = 0; k < kBwdOuts; ++k) outs[k] = o[k];
}

}  // namespace

extern "C" {

kda_status kda_validate_backward(const kda_backward_args* a) {
  if (a == nullptr) return KDA_ERR_NULL;
  const kda_prefill_args* f = &a->fwd;
  if (kda_status e = kda_validate_prefill(f); e != KDA_OK) return e;
  if ((a->dA_log || a->ddt_bias) && f->A_log == nullptr) return KDA_ERR_NULL;
  if (a->do_norm_w && f->o_norm_w == nullptr) return KDA_ERR_NULL;
  if (a->do_gate && f->o_gate == nullptr) return KDA_ERR_NULL;
  const bool need = f->T > 0;
  if (need && (!a->dO || !a->dq || !a->dk || !a->dv || !a->dg || !a->dbeta)) return KDA_ERR_NULL;
  if (f->conv_k > 0 && !a->dconv_w) return KDA_ERR_NULL;
  if (f->conv_k == 0 && (a->dconv_w || a->dconv_state)) return KDA_ERR_NULL;
  for (const void* p : std::initializer_list<const void*>{a->dO, a->dS_T, a->dq, a->dk, a->dv, a->dg,
                                                          a->dbeta, a->dS0, a->dconv_w, a->dconv_state,
                                                          a->dA_log, a->ddt_bias, a->do_norm_w,
                                                          a->do_gate})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  Span ins[kBwdIns], outs[kBwdOuts];
  bwd_spans(a, ins, outs);
  for (int i = 0; i < kBwdOuts; ++i) {
    for (int j = 0; j < kBwdIns; ++j)
      if (overlaps(outs[i], ins[j])) return KDA_ERR_ALIAS;
    for (int j = 0; j < kBwdOuts; ++j)
      if (i != j && overlaps(outs[i], outs[j])) return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

size_t kda_backward_workspace_bytes(const kda_backward_args* a) {
  if (kda_validate_backward(a) != KDA_OK) return 0;
  if (a->fwd.T == 0) return 0;
  return bwd_layout(a).bytes;
}

}  // extern "C"

// The gradients when the call has no tokens: dS0 = dS_T, the filter, history and
// stage-parameter gradients zero.
static kda_status backward_no_tokens(const kda_backward_args* a, hipStream_t st) {
  const kda_prefill_args* f = &a->fwd;
  PrefillSizes sz;
  prefill_sizes(f, sz);
  if (a->dS0 != nullptr &&
      kda::launch_copy_state(a->dS_T, a->dS0, (size_t)sz.NS * f->H * f->D * f->D, st) != hipSuccess)
    return KDA_ERR_HIP;
  if (a->dconv_w != nullptr &&
      kda::launch_copy_state(nullptr, a->dconv_w, (size_t)3 * f->H * f->D * f->conv_k, st) != hipSuccess)
    return KDA_ERR_HIP;
  if (a->dconv_state != nullptr &&
      kda::launch_copy_state(nullptr, a->dconv_state, (size_t)sz.NS * 3 * 3 * f->H * f->D, st) != hipSuccess)
    return KDA_ERR_HIP;
  // sums over no tokens
  for (auto [p, n] : {std::pair<float*, size_t>{a->dA_log, (size_t)f->H},
                      {a->ddt_bias, (size_t)f->H * f->D}, {a->do_norm_w, (size_t)f->D}})
    if (p != nullptr && kda::launch_copy_state(nullptr, p, n, st) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

// The workspace checks of a backward call with T > 0.
static kda_status check_bwd_workspace(const kda_backward_args* a, void* ws, size_t ws_bytes,
                                      const BwdLayout& L) {
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < L.bytes)
    return KDA_ERR_WORKSPACE;
  const Span w = span(ws, L.bytes);
  Span ins[kBwdIns], outs[kBwdOuts];
  bwd_spans(a, ins, outs);
  for (const Span& x : ins)
    if (overlaps(w, x)) return KDA_ERR_ALIAS;
  for (const Span& x : outs)
    if (overlaps(w, x)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

// The forward in backward mode: the mixer without the output stage, keeping in
// the workspace what the backward reads (records, front-end outputs, Gamma, beta,
// T, the state at each chunk start and U).  o then holds the mixer's output.
static kda_status forward_for_backward(const kda_prefill_args* f, char* wsb, const BwdLayout& L,
                                       hipStream_t st, BwdFwdOut& bo) {
  auto F = [&](size_t off) { return reinterpret_cast<float*>(wsb + off); };
  const kda_prefill_args f0 = forward_of_backward(f);
  bo = BwdFwdOut{wsb + L.y, F(L.gam), F(L.beta), F(L.tT), wsb + L.ckS};
  for (int stage : {KDA_STAGE_PREP, KDA_STAGE_STATE})
    if (kda_status e = run_stage(&f0, wsb, stage, st, &bo); e != KDA_OK) return e;
  return KDA_OK;
}

// Everything after the forward: the output stage's backward (from the mixer's
// output o_pre; finish_o: then the stage finishes o in place), the reverse walk
// and the per-chunk gradient kernels, the front end, the activations' backward.
static kda_status backward_core(const kda_backward_args* a, char* wsb, const BwdLayout& L,
                                const void* o_pre, bool finish_o, hipStream_t st) {
  const kda_prefill_args* f = &a->fwd;
  void* ws = wsb;
  const bool fp32 = f->io == KDA_FP32;
  PrefillSizes sz;
  prefill_sizes(f, sz);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(wsb + off); };
  const bool gn = f->o_norm_w != nullptr || f->o_gate != nullptr;
  const kda_prefill_args f0 = forward_of_backward(f);
  const void* dO = a->dO;
  if (gn) {
    kda::BwdOutParams q{};
    q.x = o_pre;
    q.z = f->o_gate;
    q.dy = a->dO;
    q.w = f->o_norm_w;
    q.eps = f->o_norm_eps;
    q.dx = wsb + L.dOp;
    q.dz = a->do_gate;
    q.dw_part = F(L.dwp);
    q.rows = (long)f->B * f->T * f->H;
    q.H = f->H;
    q.seqs = seq_tables(f, ws);
    if (kda_status e = hip_status(kda::launch_bwd_out_stage(q, a->do_norm_w, f->D, fp32, st)); e != KDA_OK)
      return e;
    if (finish_o) {
      kda::OutStageParams os{};
      os.o = f->o;
      os.o_gate = f->o_gate;
      os.o_norm_w = f->o_norm_w;
      os.o_norm_eps = f->o_norm_eps;
      os.rows = q.rows;
      if (kda_status e = hip_status(kda::launch_out_stage(os, f->D, fp32, st)); e != KDA_OK) return e;
    }
    dO = wsb + L.dOp;
  }
  // backward
  const kda::SeqTables seqs = seq_tables(f, ws);  // packed: written by the preparation above
  int* fstart = nullptr;
  if (packed(f)) {
    // the same bounds and chunk slots again, plus each sequence's first block slot
    // of the backward front end
    kda::IndexParams ip{};
    ip.cu_seqlens = f->cu_seqlens;
    ip.bounds = const_cast<int*>(seqs.bounds);
    ip.cstart = const_cast<int*>(seqs.cstart);
    ip.n_seqs = f->n_seqs;
    ip.T = f->T;
    ip.C = f->chunk;
    ip.fstart = fstart = reinterpret_cast<int*>(wsb + L.fst);
    ip.FB = kda::bwd_front_tokens(f->D);
    if (kda_status e = hip_status(kda::launch_seq_index(ip, st)); e != KDA_OK) return e;
  }
  kda::BwdLaunch B{};
  const char* recs = wsb + ws_layout(&f0).records;
  B.walk.ws = recs;
  B.walk.dO = dO;
  B.walk.dS_T = a->dS_T;
  B.walk.dS0 = a->dS0;
  B.walk.dU = wsb + L.dU;
  B.walk.ckdS = wsb + L.ckdS;
  B.walk.B = sz.NS; B.walk.T = f->T; B.walk.H = f->H; B.walk.NT = sz.NT;  // one walk per sequence
  B.walk.seqs = seqs;
  // split as the forward walk above was: its maps M are the reverse walk's too
  if (const SplitPlan sp = split_plan(&f0); sp.nseg > 1) {
    B.walk.nseg = sp.nseg;
    B.walk.seg_len = sp.seg_len;
    B.walk.maps = reinterpret_cast<float*>(wsb + ws_layout(&f0).split);
    B.walk.starts = B.walk.maps + (size_t)f->B * f->H * (sp.nseg - 1) * 3 * f->D * f->D;
  }
  B.prod.ws = recs;
  B.prod.dO = dO;
  B.prod.ckS = wsb + L.ckS;
  B.prod.ckdS = wsb + L.ckdS;
  B.prod.dU = wsb + L.dU;
  B.prod.dQL = F(L.dQL); B.prod.dW = F(L.dW); B.prod.dKt = F(L.dKt); B.prod.dP = F(L.dP);
  B.prod.dLC = F(L.dLC);
  B.prod.B = f->B; B.prod.T = f->T; B.prod.H = f->H; B.prod.NT = sz.NT;
  B.prod.seqs = seqs;
  B.tside.tT = F(L.tT);
  B.tside.y = wsb + L.y; B.tside.gam = F(L.gam); B.tside.beta = F(L.beta);
  B.tside.dW = F(L.dW); B.tside.dU = wsb + L.dU;
  B.tside.dBk = F(L.dBk); B.tside.dBv = F(L.dBv); B.tside.dA = F(L.dA);
  B.tside.B = f->B; B.tside.T = f->T; B.tside.H = f->H; B.tside.NT = sz.NT;
  B.tside.seqs = seqs;
  B.pair.y = wsb + L.y; B.pair.gam = F(L.gam); B.pair.beta = F(L.beta);
  B.pair.dA = F(L.dA); B.pair.dP = F(L.dP); B.pair.dQL = F(L.dQL); B.pair.dKt = F(L.dKt);
  B.pair.dLC = F(L.dLC); B.pair.dBk = F(L.dBk); B.pair.dBv = F(L.dBv);
  B.pair.dy = wsb + L.dy; B.pair.dg = a->dg; B.pair.dbeta_part = F(L.dbp);
  B.pair.ex_count = reinterpret_cast<unsigned*>(wsb + L.pl);
  B.pair.ex_list = B.pair.ex_count + 64;
  B.pair.B = f->B; B.pair.T = f->T; B.pair.H = f->H; B.pair.NT = sz.NT;
  B.pair.seqs = seqs;
  B.front.q = f->q; B.front.k = f->k; B.front.v = f->v;
  B.front.conv_w = f->conv_k > 0 ? f->conv_w : nullptr;
  B.front.conv_state_in = f->conv_k > 0 ? f->conv_state_in : nullptr;
  B.front.dy = wsb + L.dy;
  B.front.dq = a->dq; B.front.dk = a->dk; B.front.dv = a->dv;
  B.front.dconv_part = f->conv_k > 0 ? F(L.dcp) : nullptr;
  B.front.dconv_state = a->dconv_state;
  B.front.B = f->B; B.front.T = f->T; B.front.H = f->H;
  B.front.l2 = (f->flags & KDA_FLAG_L2NORM_QK) ? 1 : 0;
  B.front.eps = f->l2_eps;
  B.front.scale = f->scale;
  B.front.seqs = seqs;
  B.front.fstart = fstart;
  B.front.nfslots = packed(f) ? (int)L.nfront : 0;
  B.dbeta = a->dbeta;
  B.dconv_w = a->dconv_w;
  if (kda_status e = hip_status(kda::launch_backward(B, f->D, f->chunk, fp32, st)); e != KDA_OK)
    return e;
  if (packed(f) && f->conv_k > 0 &&
      hip_status(kda::launch_bwd_empty_history(a->dconv_state, seqs.bounds, f->n_seqs,
                                               (long)3 * (f->conv_k - 1) * f->H * f->D, st)) != KDA_OK)
    return KDA_ERR_HIP;
  const bool logits = (f->flags & KDA_FLAG_BETA_LOGITS) != 0;
  if (f->A_log != nullptr || logits) {
    kda::BwdActParams q{};
    q.f = f->A_log != nullptr ? f->g : nullptr;
    q.A_log = f->A_log;
    q.dt_bias = f->dt_bias;
    q.dg = a->dg;
    q.ddt_part = F(L.ddp);
    q.dA_part = F(L.dap);
    q.beta = logits ? F(L.beta) : nullptr;
    q.dbeta = a->dbeta;
    q.tokens = (long)f->B * f->T;
    q.H = f->H;
    q.seqs = seqs;
    if (kda_status e = hip_status(kda::launch_bwd_act(q, a->dA_log, a->ddt_bias, f->D, fp32, st));
        e != KDA_OK)
      return e;
  }
  return KDA_OK;
}

extern "C" {

kda_status kda_prefill_backward(const kda_backward_args* a, void* ws, size_t ws_bytes, void* stream) {
  if (kda_status e = kda_validate_backward(a); e != KDA_OK) return e;
  const kda_prefill_args* f = &a->fwd;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (f->T == 0) {
    if (kda_status e = backward_no_tokens(a, st); e != KDA_OK) return e;
    // the run_stage calls below still hand S_T and the conv state through
    for (int stage = KDA_STAGE_PREP; stage <= KDA_STAGE_OUTPUT; ++stage)
      if (kda_status e = run_stage(f, ws, stage, st); e != KDA_OK) return e;
    return KDA_OK;
  }
  const BwdLayout L = bwd_layout(a);
  if (kda_status e = check_bwd_workspace(a, ws, ws_bytes, L); e != KDA_OK) return e;
  char* wsb = static_cast<char*>(ws);
  // The conv-state hand-over comes last, after the backward front end has read the
  // previous conv state: conv_state_out may be conv_state_in, and the hand-over
  // overwrites it.  With the output stage the walk leaves the mixer's output in o;
  // the stage's backward reads it, then the stage finishes o in place.
  BwdFwdOut bo{};
  if (kda_status e = forward_for_backward(f, wsb, L, st, bo); e != KDA_OK) return e;
  if (kda_status e = backward_core(a, wsb, L, f->o, true, st); e != KDA_OK) return e;
  return run_stage(f, ws, KDA_STAGE_CONV_TAIL, st, &bo);
}

// The saved forward's workspace: the backward's, plus the mixer's output before
// the output stage when there is one.
static kda_backward_args backward_of_forward(const kda_prefill_args* f) {
  kda_backward_args b{};
  b.fwd = *f;
  return b;
}

size_t kda_training_workspace_bytes(const kda_prefill_args* f) {
  if (kda_validate_prefill(f) != KDA_OK || f->T == 0) return 0;
  const kda_backward_args b = backward_of_forward(f);
  return bwd_layout(&b, true).bytes;
}

kda_status kda_prefill_forward_saved(const kda_prefill_args* f, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (kda_status e = kda_validate_prefill(f); e != KDA_OK) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (f->T == 0) {
    for (int stage = KDA_STAGE_PREP; stage <= KDA_STAGE_OUTPUT; ++stage)
      if (kda_status e = run_stage(f, ws, stage, st); e != KDA_OK) return e;
    return KDA_OK;
  }
  PrefillSizes sz;
  prefill_sizes(f, sz);
  // the backward reads the previous conv state after this call has written the new one
  if (overlaps(span(f->conv_state_in, sz.cst), span(f->conv_state_out, sz.cst))) return KDA_ERR_ALIAS;
  const kda_backward_args b = backward_of_forward(f);
  const BwdLayout L = bwd_layout(&b, true);
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < L.bytes)
    return KDA_ERR_WORKSPACE;
  const Span w = span(ws, L.bytes);
  for (Span x : {span(f->q, sz.x), span(f->k, sz.x), span(f->v, sz.x), span(f->g, sz.x),
                 span(f->beta, sz.bta), span(f->conv_w, sz.cw), span(f->conv_state_in, sz.cst),
                 span(f->S0, sz.state), span(f->o, sz.x), span(f->S_T, sz.state),
                 span(f->conv_state_out, sz.cst), span(f->A_log, (size_t)f->H * 4),
                 span(f->dt_bias, (size_t)f->H * f->D * 4), span(f->o_norm_w, (size_t)f->D * 4),
                 span(f->o_gate, sz.x), span(f->cu_seqlens, sz.cu)})
    if (overlaps(w, x)) return KDA_ERR_ALIAS;
  char* wsb = static_cast<char*>(ws);
  BwdFwdOut bo{};
  if (kda_status e = forward_for_backward(f, wsb, L, st, bo); e != KDA_OK) return e;
  if (f->o_norm_w != nullptr || f->o_gate != nullptr) {
    // keep the mixer's output for the output stage's backward, then finish o
    if (kda::launch_copy_state(static_cast<const float*>(f->o), reinterpret_cast<float*>(wsb + L.opre),
                               sz.x / 4, st) != hipSuccess)
      return KDA_ERR_HIP;
    kda::OutStageParams os{};
    os.o = f->o;
    os.o_gate = f->o_gate;
    os.o_norm_w = f->o_norm_w;
    os.o_norm_eps = f->o_norm_eps;
    os.rows = (long)f->B * f->T * f->H;
    if (kda_status e = hip_status(kda::launch_out_stage(os, f->D, f->io == KDA_FP32, st)); e != KDA_OK)
      return e;
  }
  return run_stage(f, ws, KDA_STAGE_CONV_TAIL, st, &bo);
}

kda_status kda_prefill_backward_saved(const kda_backward_args* a, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (kda_status e = kda_validate_backward(a); e != KDA_OK) return e;
  const kda_prefill_args* f = &a->fwd;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (f->T == 0) return backward_no_tokens(a, st);
  PrefillSizes sz;
  prefill_sizes(f, sz);
  if (overlaps(span(f->conv_state_in, sz.cst), span(f->conv_state_out, sz.cst))) return KDA_ERR_ALIAS;
  const BwdLayout L = bwd_layout(a, true);
  if (kda_status e = check_bwd_workspace(a, ws, ws_bytes, L); e != KDA_OK) return e;
  char* wsb = static_cast<char*>(ws);
  return backward_core(a, wsb, L, wsb + L.opre, false, st);
}

}  // extern "C"
