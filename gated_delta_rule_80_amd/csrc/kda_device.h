// Device helpers for the KDA kernels on gfx950 (CDNA4): element conversions,
// 16x16 matrix-core tiles and small wave utilities.
//
// Matrix-core tile convention used everywhere (wave64, 16 x 16 output tile):
//   operand rows:  lane l supplies row (l % 16) of the A operand and column
//                  (l % 16) of the B operand, with a run of consecutive k values
//                  chosen by the lane group g = l / 16.  A and B use the same
//                  (g, slot) -> k assignment, so the contraction is over the full
//                  k range whatever order the hardware walks it in.
//   accumulator:   lane l holds column (l % 16), rows 4*(l/16) + 0..3.
// Both operands are read "along k": A as rows of A, B as rows of B^T.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Address-space-qualified pointers for the direct global-to-LDS copy builtin.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // RNE

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as floats.
__device__ __forceinline__ void load8(const __bf16* p, float* out) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(__bf16* p, const float* in) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)in[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float* in) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = in[i]; b[i] = in[4 + i]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}
// 4 consecutive elements as float32 (8-byte aligned bf16 / 16-byte aligned fp32)
// 4 elements of type E as one vector (bf16x4 / f32x4)
template <typename E> struct Vec4;
template <> struct Vec4<__bf16> { using type = bf16x4; };
template <> struct Vec4<float> { using type = f32x4; };

__device__ __forceinline__ f32x4 load4v(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4v(const __bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// 4 consecutive elements (8-byte aligned bf16 / 16-byte aligned fp32)
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}
// 2 consecutive elements (4-byte aligned bf16 / 8-byte aligned fp32)
__device__ __forceinline__ void store2(__bf16* p, float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b;
  *reinterpret_cast<bf16x2*>(p) = v;
}
__device__ __forceinline__ void store2(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void load4(const __bf16* p, float* out) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
}
__device__ __forceinline__ void load4(const float* p, float* out) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}

// ------------------------------------------------------------ matrix-core tiles
// A 16-deep bf16 product step (4 k-values per lane) issued as the 32-deep
// instruction with the other 4 k-slots zero on both sides.  Every bf16 product
// then uses one instruction shape, so dependent accumulation chains never mix
// shapes.
__device__ __forceinline__ f32x4 mfma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 acc) {
  const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
  const bf16x8 a8 = __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8 b8 = __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
}

// acc(16x16) += A(16 x K) * B(K x 16) where A is given by its rows (A + m*lda, k
// contiguous) and B by the rows of B^T (Bt + n*ldb, k contiguous).  K is a
// compile-time multiple of 16 (bf16) or 4 (fp32).  Pointers may be LDS or global.
template <int K>
__device__ __forceinline__ void mma_rows(f32x4& acc, const __bf16* A, int lda, const __bf16* Bt,
                                         int ldb, int lane) {
  const int r = lane & 15, g = lane >> 4;
  static_assert(K % 16 == 0, "bf16 tiles need K % 16 == 0");
  if constexpr (K % 32 == 0) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k0 + 8 * g);
      bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k0 + 8 * g);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
      bf16x4 a = *reinterpret_cast<const bf16x4*>(A + r * lda + k0 + 4 * g);
      bf16x4 b = *reinterpret_cast<const bf16x4*>(Bt + r * ldb + k0 + 4 * g);
      acc = mfma_bf16_k16(a, b, acc);
    }
  }
}
template <int K>
__device__ __forceinline__ void mma_rows(f32x4& acc, const float* A, int lda, const float* Bt,
                                         int ldb, int lane) {
  const int r = lane & 15, g = lane >> 4;
  static_assert(K % 4 == 0, "fp32 tiles need K % 4 == 0");
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + g], Bt[r * ldb + k0 + g], acc, 0,
                                               0, 0);
  }
}

// Same as mma_rows but only over k in [0, kmax) rounded up to the instruction
// depth (kmax is a runtime bound used for causal skipping; entries past the true
// bound must be zero in memory or masked by the caller).
template <int K>
__device__ __forceinline__ void mma_rows_upto(f32x4& acc, const __bf16* A, int lda,
                                              const __bf16* Bt, int ldb, int lane, int kmax) {
  const int r = lane & 15, g = lane >> 4;
  if constexpr (K % 32 == 0) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      if (k0 < kmax) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k0 + 8 * g);
        bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + r * ldb + k0 + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
      if (k0 < kmax) {
        bf16x4 a = *reinterpret_cast<const bf16x4*>(A + r * lda + k0 + 4 * g);
        bf16x4 b = *reinterpret_cast<const bf16x4*>(Bt + r * ldb + k0 + 4 * g);
        acc = mfma_bf16_k16(a, b, acc);
      }
    }
  }
}
template <int K>
__device__ __forceinline__ void mma_rows_upto(f32x4& acc, const float* A, int lda, const float* Bt,
                                              int ldb, int lane, int kmax) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4) {
    if (k0 < kmax)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + g], Bt[r * ldb + k0 + g], acc, 0,
                                                 0, 0);
  }
}

// One lane's share of a 16-row matrix-core operand over a compile-time depth K,
// read "along k" from row (base + (l % 16) * ld).  The same registers serve as
// the A operand (rows of A) or the B operand (rows of B^T).
template <typename E, int K> struct RowFrag;

template <int K> struct RowFrag<__bf16, K> {
  static constexpr bool X32 = (K % 32) == 0;
  static constexpr int STEP = X32 ? 32 : 16;
  static constexpr int PER = X32 ? 8 : 4;  // elements per lane per step
  static constexpr int N = K / STEP;
  static_assert(K % 16 == 0, "bf16 operands need K % 16 == 0");
  using V = typename std::conditional<X32, bf16x8, bf16x4>::type;
  V v[N];
  // row: pointer to this lane's row (row 0 of the tile + (lane % 16) * ld)
  __device__ __forceinline__ void load(const __bf16* row, int g) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = *reinterpret_cast<const V*>(row + i * STEP + PER * g);
  }
  // zero every element whose k index exceeds kmax (causal mask)
  __device__ __forceinline__ void mask_above(int kmax, int g) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (i * STEP + PER * g + e > kmax) v[i][e] = (__bf16)0.f;
  }
  // zero every element whose k index is below kmin
  __device__ __forceinline__ void mask_below(int kmin, int g) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (i * STEP + PER * g + e < kmin) v[i][e] = (__bf16)0.f;
  }
};

template <int K> struct RowFrag<float, K> {
  static constexpr int STEP = 4;
  static constexpr int N = K / 4;
  static_assert(K % 4 == 0, "fp32 operands need K % 4 == 0");
  float v[N];
  __device__ __forceinline__ void load(const float* row, int g) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = row[4 * i + g];
  }
  __device__ __forceinline__ void mask_above(int kmax, int g) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (4 * i + g > kmax) v[i] = 0.f;
  }
  __device__ __forceinline__ void mask_below(int kmin, int g) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (4 * i + g < kmin) v[i] = 0.f;
  }
};

// acc += A * B over the first `steps` k-steps (all by default)
template <int K>
__device__ __forceinline__ void mma(f32x4& acc, const RowFrag<__bf16, K>& a,
                                    const RowFrag<__bf16, K>& b, int steps = RowFrag<__bf16, K>::N) {
#pragma unroll
  for (int i = 0; i < RowFrag<__bf16, K>::N; ++i) {
    if (i < steps) {
      if constexpr (RowFrag<__bf16, K>::X32) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[i], b.v[i], acc, 0, 0, 0);
      } else {
        acc = mfma_bf16_k16(a.v[i], b.v[i], acc);
      }
    }
  }
}
template <int K>
__device__ __forceinline__ void mma(f32x4& acc, const RowFrag<float, K>& a,
                                    const RowFrag<float, K>& b, int steps = RowFrag<float, K>::N) {
#pragma unroll
  for (int i = 0; i < RowFrag<float, K>::N; ++i)
    if (i < steps) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// ------------------------------------------------- swizzled LDS matrix images
// A row-major matrix of K elements per row stored in LDS with its 16-byte chunks
// permuted within each row: chunk c of row `row` sits at position c ^ (row % RC),
// RC = chunks per row.  Sixteen lanes reading the same k range of 16 different
// rows then hit distinct banks.
template <typename E, int K>
struct Swz {
  static constexpr int EPC = 16 / (int)sizeof(E);  // elements per chunk
  static constexpr int RC = K / EPC;               // chunks per row (power of two)
  static_assert(RC >= 1 && (RC & (RC - 1)) == 0, "rows must hold a power-of-two chunk count");
  // element offset of element k of `row`
  __device__ __forceinline__ static int at(int row, int k) {
    return row * K + (((k / EPC) ^ (row & (RC - 1))) * EPC) + (k % EPC);
  }
};

// Load this lane's fragment of row `row` from a swizzled LDS image.
template <int K>
__device__ __forceinline__ void load_swz(RowFrag<__bf16, K>& f, const __bf16* img, int row, int g) {
  using FR = RowFrag<__bf16, K>;
#pragma unroll
  for (int i = 0; i < FR::N; ++i)
    f.v[i] = *reinterpret_cast<const typename FR::V*>(img + Swz<__bf16, K>::at(row, i * FR::STEP + FR::PER * g));
}
template <int K>
__device__ __forceinline__ void load_swz(RowFrag<float, K>& f, const float* img, int row, int g) {
#pragma unroll
  for (int i = 0; i < RowFrag<float, K>::N; ++i) f.v[i] = img[Swz<float, K>::at(row, 4 * i + g)];
}

// Transposed fragment: this lane's fragment of column j of a swizzled image with
// KM elements per row (the fragment's k runs over the image's rows, KF of them).
template <int KF, int KM>
__device__ __forceinline__ void load_swz_t(RowFrag<__bf16, KF>& f, const __bf16* img, int j, int g) {
  using FR = RowFrag<__bf16, KF>;
#pragma unroll
  for (int i = 0; i < FR::N; ++i)
#pragma unroll
    for (int e = 0; e < FR::PER; ++e)
      f.v[i][e] = img[Swz<__bf16, KM>::at(i * FR::STEP + FR::PER * g + e, j)];
}
template <int KF, int KM>
__device__ __forceinline__ void load_swz_t(RowFrag<float, KF>& f, const float* img, int j, int g) {
#pragma unroll
  for (int i = 0; i < RowFrag<float, KF>::N; ++i) f.v[i] = img[Swz<float, KM>::at(4 * i + g, j)];
}

// The same transposed bf16 fragment with gfx950's transposing LDS read
// (ds_read_b64_tr_b16).  Within each group of 16 lanes, output lane i element e is
// element i % 4 of the 8 bytes lane 4 e + i / 4 addressed; so lane r of the group
// addresses image row k0 + r / 4, columns m0 + 4 (r % 4) .. + 3, and receives
// column m0 + r of rows k0 .. k0 + 3: four k-elements of its fragment in one read.
// The lanes of a group share g (lanes 16 g .. 16 g + 15), m0 is the fragment's
// 16-column block of the image, r the lane's index within its group.  A lane's
// result comes from the addresses of other lanes of its group, so all 16 must be
// active: call it from wave-uniform control flow only.
template <int KF, int KM>
__device__ __forceinline__ void load_swz_tr(RowFrag<__bf16, KF>& f, const __bf16* img, int m0, int r,
                                            int g) {
  using FR = RowFrag<__bf16, KF>;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int col = m0 + 4 * (r & 3);
#pragma unroll
  for (int i = 0; i < FR::N; ++i)
#pragma unroll
    for (int hh = 0; hh < FR::PER / 4; ++hh) {
      const int row = i * FR::STEP + FR::PER * g + 4 * hh + (r >> 2);
      // (the bf16 form of the builtin: the 16-bit integer form with each element
      // cast to bf16 was compiled to use element 0 four times)
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(img + Swz<__bf16, KM>::at(row, col)));
#pragma unroll
      for (int e = 0; e < 4; ++e) f.v[i][4 * hh + e] = v[e];
    }
}
// Transposed fragment of column m0 + r: the transposing read for bf16, element
// reads for fp32 (which has no such read).
template <int KF, int KM>
__device__ __forceinline__ void load_frag_t(RowFrag<__bf16, KF>& f, const __bf16* img, int m0, int r,
                                            int g) {
  load_swz_tr<KF, KM>(f, img, m0, r, g);
}
template <int KF, int KM>
__device__ __forceinline__ void load_frag_t(RowFrag<float, KF>& f, const float* img, int m0, int r,
                                            int g) {
  load_swz_t<KF, KM>(f, img, m0 + r, g);
}

// Instruction depth along k for an element type (used for causal bounds).
template <typename E> struct KStep;
template <> struct KStep<__bf16> { static constexpr int value = 32; };
template <> struct KStep<float> { static constexpr int value = 4; };

// Workgroup barrier ordering LDS accesses only: waits for this wave's LDS
// operations, not for its outstanding global-memory operations (including
// global-to-LDS copies into a buffer nobody touches until a later full barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Vector memory operations retire
// in issue order, so this waits for everything but the N most recent ones.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Position of workgroup blk of an n-workgroup grid in the order that lists the
// workgroups XCD by XCD.  Dispatch places workgroup blk on XCD blk % 8, so the
// positions [x (n / 8) + min(x, n % 8), ...) all run on XCD x and consecutive
// positions share that XCD's L2 (up to the 7 boundaries between XCDs).
__device__ __forceinline__ int xcd_major(int blk, int n) {
  const int x = blk & 7, i = blk >> 3, q = n >> 3, rem = n & 7;
  return x * q + (x < rem ? x : rem) + i;
}

// ------------------------------------------------------------ packed sequences
// The sequence that owns chunk slot gc: the largest i < n_seqs with cstart[i] <=
// gc (an empty sequence owns no slot, so it is skipped).  gc < cstart[n_seqs].
__device__ __forceinline__ int seq_of_slot(const int* cstart, int n_seqs, int gc) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cstart[mid] <= gc)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------ small math
__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }
// ln(1 + e^x) as max(x, 0) + ln(1 + e^-|x|) with the hardware exp and log: no
// overflow; where e^-|x| < 2^-24 the second term rounds to 0, an absolute error
// below 6e-8 (the decay of such a channel is below 1e-7 per token anyway).
__device__ __forceinline__ float softplus(float x) {
  return fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x)));
}
// Log-decay of one key channel from the raw gate projection f: -exp(A_log[h]) *
// softplus(f + dt_bias[c]); `neg_rate` is -exp(A_log[h]) (times any unit change).
__device__ __forceinline__ float gate_decay(float f, float bias, float neg_rate) {
  return neg_rate * softplus(f + bias);
}

// x from another lane of the same 16-lane row by a DPP lane pattern (all lanes
// active)
template <int CTRL>
__device__ __forceinline__ float dpp_get(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                            0xF, false));
}

// Sum over groups of `W` consecutive lanes (W a power of two <= 64), every lane
// of a group receiving the group's sum.  Groups of up to 16 lanes use DPP lane
// patterns inside a row, each pairing lanes from different halves of the
// current partial group: swap neighbours, swap pairs (quad_perm), mirror the 8
// lanes of a half row, mirror the row.  Wider groups add xor-shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "power-of-two group");
  if constexpr (W >= 2) x += dpp_get<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) x += dpp_get<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) x += dpp_get<0x141>(x);  // row_half_mirror
  if constexpr (W >= 16) x += dpp_get<0x140>(x); // row_mirror
#pragma unroll
  for (int m = 16; m < W; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

}  // namespace kda
