// kda_common.hpp -- device building blocks shared by the gfx950 KDA kernels.
//
// Conventions
//  * Chunk length CH = 64 tokens.  A "chunk-head" is one chunk of one head.
//  * MFMA tiles are 16x16 with a 32-deep contraction (v_mfma_f32_16x16x32_bf16,
//    or eight v_mfma_f32_16x16x4_f32 for the fp32 path).  In a wave, lane l
//    supplies row/column (l & 15) of an operand and the 8 consecutive
//    contraction indices 8*(l >> 4) .. +7; it receives the accumulator
//    elements (row 4*(l >> 4) + i, column l & 15), i = 0..3.  A and B use the
//    same lane->k assignment, so the product is exact whatever order the
//    hardware sums the 32 terms in.
//  * LDS operand arrays are stored "k-contiguous" where possible so one
//    fragment is one 16-byte LDS read; rows are padded by 16 bytes to spread
//    banks.  frag_col() reads a fragment from the other orientation with
//    eight scalar reads (used where a second copy would cost more LDS).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

constexpr int CH = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // raw 16-byte vector (native, so it stays in registers)

// MFMA operand type of the intermediates for a given input type: fp16 for bf16
// inputs (11-bit significand, same MFMA rate as bf16; every intermediate it
// carries is bounded by the inputs' magnitudes), fp32 for the fp32 path.
template <typename E> struct OpOf { using T = f16; };
template <> struct OpOf<float> { using T = float; };

struct ChunkInfo {
  int32_t seq;  // sequence index
  int32_t t0;   // first packed token of the chunk
  int32_t len;  // valid tokens (0 => unused slot)
  int32_t idx;  // chunk index inside its sequence
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Small lists of 2-bit values packed into one 64-bit word: a lookup with a run-time
// index is then a shift in registers.  (A constexpr array indexed at run time is
// placed in global memory, and the wait for its load also waits for every vector
// load and store the wave still has in flight.)
template <int N>
__host__ __device__ constexpr uint64_t pack2(const int (&v)[N]) {
  static_assert(N <= 32, "at most 32 entries");
  uint64_t p = 0;
  for (int i = 0; i < N; ++i) p |= (uint64_t)(v[i] & 3) << (2 * i);
  return p;
}
__device__ __forceinline__ int unpack2(uint64_t p, int i) { return (int)((p >> (2 * i)) & 3); }

__device__ __forceinline__ float f32(float x) { return x; }
__device__ __forceinline__ float f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float f32(f16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E cvt(float x);
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 cvt<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ f16 cvt<f16>(float x) { return (f16)x; }     // RNE

// Sums over aligned groups of 8 or 16 consecutive lanes, every lane of the group
// receiving the group's total.  DPP lane permutes inside a 16-lane row (swap
// neighbours, swap pairs, mirror each half-row, mirror the row) are plain vector ALU
// operations, where a shuffle would go through the LDS crossbar; every lane of the wave
// must be active.
template <int CTRL> __device__ __forceinline__ float dpp_take(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_sum8(float v) {
  v += dpp_take<0xB1>(v);    // quad_perm [1, 0, 3, 2]: lane ^ 1
  v += dpp_take<0x4E>(v);    // quad_perm [2, 3, 0, 1]: lane ^ 2
  v += dpp_take<0x141>(v);   // row_half_mirror: lane i <-> 7 - i, so each quad meets the other
  return v;
}
__device__ __forceinline__ float lane_sum16(float v) {
  v = lane_sum8(v);
  v += dpp_take<0x140>(v);   // row_mirror: lane i <-> 15 - i, so each half-row meets the other
  return v;
}

// 4x4 transpose across each quad of lanes (lanes 4g .. 4g + 3): lane 4g + c holds
// x[r] = M[r][c] and receives x[c] = M[lane & 3][c].  Two exchange stages, across lane ^ 1
// and lane ^ 2, each trade the two values whose register bit differs from the lane bit.
// Used to turn an MFMA output tile (a lane holds four rows of one column) into four
// consecutive columns of one row for a 16-byte store.  Every lane of the wave must be active.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x) {
  const int i = (int)threadIdx.x & 3;
  {
    const bool odd = i & 1;
    float s0 = odd ? x[0] : x[1], s1 = odd ? x[2] : x[3];
    s0 = dpp_take<0xB1>(s0);   // lane ^ 1
    s1 = dpp_take<0xB1>(s1);
    if (odd) {
      x[0] = s0;
      x[2] = s1;
    } else {
      x[1] = s0;
      x[3] = s1;
    }
  }
  {
    const bool hi = i & 2;
    float s0 = hi ? x[0] : x[2], s1 = hi ? x[1] : x[3];
    s0 = dpp_take<0x4E>(s0);   // lane ^ 2
    s1 = dpp_take<0x4E>(s1);
    if (hi) {
      x[0] = s0;
      x[1] = s1;
    } else {
      x[2] = s0;
      x[3] = s1;
    }
  }
  return x;
}

// Row padding of LDS arrays, in elements (16 bytes).
template <typename E> constexpr int PADE = 16 / (int)sizeof(E);

// ---------------------------------------------------------------------------
// fragments and MFMA
// ---------------------------------------------------------------------------
template <typename E> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<f16> { f16x8 v; };
template <> struct Frag<float> { float v[8]; };

// 8 consecutive elements p[row*ld + k0 .. +7]; (row*ld + k0) must be a multiple of 16/sizeof(E)/... 16B aligned.
template <typename E> __device__ __forceinline__ Frag<E> frag_row(const E* p, int ld, int row, int k0);
template <> __device__ __forceinline__ Frag<bf16> frag_row<bf16>(const bf16* p, int ld, int row, int k0) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p + row * ld + k0);
  return f;
}
template <> __device__ __forceinline__ Frag<f16> frag_row<f16>(const f16* p, int ld, int row, int k0) {
  Frag<f16> f;
  f.v = *reinterpret_cast<const f16x8*>(p + row * ld + k0);
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_row<float>(const float* p, int ld, int row, int k0) {
  Frag<float> f;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + row * ld + k0);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + row * ld + k0 + 4);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
  return f;
}
// 8 elements down a column: p[(k0+j)*ld + col], j = 0..7.
template <typename E> __device__ __forceinline__ Frag<E> frag_col(const E* p, int ld, int col, int k0) {
  Frag<E> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = p[(k0 + j) * ld + col];
  return f;
}
// Fragment built from 8 float values (converted to the operand type).
template <typename E> __device__ __forceinline__ Frag<E> frag_from(const float (&x)[8]) {
  Frag<E> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = cvt<E>(x[j]);
  return f;
}

__device__ __forceinline__ f32x4 mma(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<f16>& a, const Frag<f16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// split operands: an fp32 value carried as x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi); a product of two split operands drops only lo*lo, so its
// error is ~2^-16 relative instead of 2^-8.  On the fp32 path the "split"
// operand is just the fp32 value (lo unused) and every product is one MFMA.
// ---------------------------------------------------------------------------
template <typename E> struct SFrag { Frag<E> hi, lo; };

template <typename E> __device__ __forceinline__ SFrag<E> sfrag_from(const float (&x)[8]) {
  SFrag<E> s;
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const E h = (E)x[j];
      s.hi.v[j] = h;
      s.lo.v[j] = (E)(x[j] - (float)h);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) s.hi.v[j] = x[j];
  }
  return s;
}
// 8 consecutive fp32 values of LDS row `row`, split.
template <typename E> __device__ __forceinline__ SFrag<E> sfrag_row(const float* p, int ld, int row, int k0) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + row * ld + k0);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + row * ld + k0 + 4);
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return sfrag_from<E>(x);
}
// hi/lo halves already stored as two E arrays of the same layout.
template <typename E> __device__ __forceinline__ SFrag<E> sfrag_pair(const E* hi, const E* lo, int ld, int row, int k0) {
  SFrag<E> s;
  s.hi = frag_row<E>(hi, ld, row, k0);
  if constexpr (sizeof(E) == 2) s.lo = frag_row<E>(lo, ld, row, k0);
  return s;
}
// 8 consecutive-k elements down a column of hi/lo arrays stored [k][col].
template <typename E> __device__ __forceinline__ SFrag<E> sfrag_col_pair(const E* hi, const E* lo, int ld, int col, int k0) {
  SFrag<E> s;
  s.hi = frag_col<E>(hi, ld, col, k0);
  if constexpr (sizeof(E) == 2) s.lo = frag_col<E>(lo, ld, col, k0);
  return s;
}
// 8 consecutive-k fp32 values down a column [k][col], split.
template <typename E> __device__ __forceinline__ SFrag<E> sfrag_col_f32(const float* p, int ld, int col, int k0) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = p[(k0 + j) * ld + col];
  return sfrag_from<E>(x);
}
// The fragment, or zeros when !keep (per lane: masks the operand rows a lane supplies).
template <typename E> __device__ __forceinline__ SFrag<E> sfrag_keep(const SFrag<E>& s, bool keep) {
  SFrag<E> z;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    z.hi.v[j] = keep ? s.hi.v[j] : (E)0.f;
    if constexpr (sizeof(E) == 2) z.lo.v[j] = keep ? s.lo.v[j] : (E)0.f;
  }
  return z;
}
template <typename E> __device__ __forceinline__ f32x4 mma_ss(const SFrag<E>& a, const SFrag<E>& b, f32x4 c) {
  if constexpr (sizeof(E) == 2) {
    c = mma(a.lo, b.hi, c);
    c = mma(a.hi, b.lo, c);
  }
  return mma(a.hi, b.hi, c);
}
template <typename E> __device__ __forceinline__ f32x4 mma_sp(const SFrag<E>& a, const Frag<E>& b, f32x4 c) {
  if constexpr (sizeof(E) == 2) c = mma(a.lo, b, c);
  return mma(a.hi, b, c);
}
template <typename E> __device__ __forceinline__ f32x4 mma_ps(const Frag<E>& a, const SFrag<E>& b, f32x4 c) {
  if constexpr (sizeof(E) == 2) c = mma(a, b.lo, c);
  return mma(a, b.hi, c);
}
// Write 4 fp32 values as a split pair into two E arrays (contiguous 4 elements each).
template <typename E> __device__ __forceinline__ void store4_split(E* hi, E* lo, float a, float b, float c, float d) {
  if constexpr (sizeof(E) == 2) {
    typedef E v4 __attribute__((ext_vector_type(4)));
    const E ha = (E)a, hb = (E)b, hc = (E)c, hd = (E)d;
    *reinterpret_cast<v4*>(hi) = v4{ha, hb, hc, hd};
    *reinterpret_cast<v4*>(lo) = v4{(E)(a - (float)ha), (E)(b - (float)hb), (E)(c - (float)hc), (E)(d - (float)hd)};
  } else {
    *reinterpret_cast<f32x4*>(hi) = f32x4{a, b, c, d};
  }
}

// C(16x16) += A(m0.., k) * B(k, n0..), contraction length K (multiple of 32).
// Operands come from LDS through loaders: la(row_in_tile, k) / lb(col_in_tile, k).
template <int K, typename LA, typename LB>
__device__ __forceinline__ f32x4 tile_mm(LA la, LB lb, f32x4 acc) {
  const int l = lane_id(), r16 = l & 15, kq = (l >> 4) * 8;
#pragma unroll
  for (int k = 0; k < K; k += 32) acc = mma(la(r16, k + kq), lb(r16, k + kq), acc);
  return acc;
}

// C(16x16) += A(m0 + ., k) * S(k, n0 + .) where A is a plain operand stored
// [m][k] and S a split operand stored as hi/lo arrays [n][k].
template <typename E, int K>
__device__ __forceinline__ f32x4 tile_mm_ps(const E* A, int lda, int m0, const E* Bh, const E* Bl, int ldb, int n0) {
  const int l = lane_id(), r16 = l & 15, kq = (l >> 4) * 8;
  f32x4 acc = zero4();
#pragma unroll
  for (int k = 0; k < K; k += 32)
    acc = mma_ps(frag_row<E>(A, lda, m0 + r16, k + kq), sfrag_pair<E>(Bh, Bl, ldb, n0 + r16, k + kq), acc);
  return acc;
}

// ---------------------------------------------------------------------------
// cooperative global <-> LDS copies (16-byte vectors)
// ---------------------------------------------------------------------------
// Copy a ROWS x COLS tile of E (row pitch src_ld elements in global, dst_ld in
// LDS) with NT threads.  COLS*sizeof(E) must be a multiple of 16.
// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N).  Register
// arrays indexed through it stay in registers (no dynamic indexing).
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, N>(f);
  }
}

template <typename E> __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d);

template <typename E, int ROWS, int COLS, int NT>
struct TileCopy {
  static constexpr int VPR = COLS * (int)sizeof(E) / 16;  // vectors per row
  static constexpr int NV = ROWS * VPR;
  static constexpr int PER = (NV + NT - 1) / NT;
  u32x4 r[PER];
  // Rows >= nrows (nrows >= 1) are not read: they re-read row 0, and a store
  // with the same nrows writes zeros there.
  __device__ __forceinline__ void load(const E* __restrict__ src, size_t src_ld, int nrows = ROWS) {
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      // threads past the tile re-read vector 0 (always in bounds) and skip the store,
      // so every register is defined on every path
      const int v0 = threadIdx.x + I * NT;
      const int v = (NV % NT == 0 || v0 < NV) ? v0 : 0;
      const int row = v / VPR, cv = v % VPR;
      const int rr = row < nrows ? row : 0;
      r[I] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src + rr * src_ld) + cv * 16);
    });
  }
  __device__ __forceinline__ void store(E* dst, int dst_ld) const {
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v = threadIdx.x + I * NT;
      if (NV % NT == 0 || v < NV) {
        const int row = v / VPR, cv = v % VPR;
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst + row * dst_ld) + cv * 16) = r[I];
      }
    });
  }
  // Store converted to D; rows >= nrows are stored as zeros.
  template <typename D>
  __device__ __forceinline__ void store_cvt(D* dst, int dst_ld, int nrows) const {
    constexpr int EPV = 16 / (int)sizeof(E);
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v = threadIdx.x + I * NT;
      if (NV % NT == 0 || v < NV) {
        const int row = v / VPR, c0 = (v % VPR) * EPV;
        const E* e = reinterpret_cast<const E*>(&r[I]);
        const bool ok = row < nrows;
#pragma unroll
        for (int i = 0; i < EPV; i += 4)
          store4<D>(dst + row * dst_ld + c0 + i, ok ? f32(e[i]) : 0.f, ok ? f32(e[i + 1]) : 0.f,
                    ok ? f32(e[i + 2]) : 0.f, ok ? f32(e[i + 3]) : 0.f);
      }
    });
  }
  // Store f(x) converted to D; rows >= nrows are stored as zeros.
  template <typename D, typename F>
  __device__ __forceinline__ void store_map(D* dst, int dst_ld, int nrows, F f) const {
    constexpr int EPV = 16 / (int)sizeof(E);
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v = threadIdx.x + I * NT;
      if (NV % NT == 0 || v < NV) {
        const int row = v / VPR, c0 = (v % VPR) * EPV;
        const E* e = reinterpret_cast<const E*>(&r[I]);
        const bool ok = row < nrows;
#pragma unroll
        for (int i = 0; i < EPV; i += 4)
          store4<D>(dst + row * dst_ld + c0 + i, ok ? f(f32(e[i])) : 0.f, ok ? f(f32(e[i + 1])) : 0.f,
                    ok ? f(f32(e[i + 2])) : 0.f, ok ? f(f32(e[i + 3])) : 0.f);
      }
    });
  }
  // fp32 tile stored as a split pair (hi, lo) of D (lo unused when D is fp32).
  // 1 / sqrt(sum x^2 + eps) of the row each held vector belongs to (the row's VPR
  // vectors sit in VPR consecutive lanes, so a butterfly over those lanes sums
  // it); the rows themselves are left as loaded.
  __device__ __forceinline__ void row_inv_norms(float eps, float (&scale)[PER]) const {
    static_assert(VPR <= 64 && (VPR & (VPR - 1)) == 0 && NT % VPR == 0, "a row spans a power-of-two lane group");
    constexpr int EPV = 16 / (int)sizeof(E);
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const E* e = reinterpret_cast<const E*>(&r[I]);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < EPV; ++i) ss += f32(e[i]) * f32(e[i]);
#pragma unroll
      for (int m = 1; m < VPR; m <<= 1) ss += __shfl_xor(ss, m);
      scale[I] = 1.0f / sqrtf(ss + eps);
    });
  }
  // Thread that writes row `row`'s entry of a per-row array (the first lane of its group).
  __device__ __forceinline__ bool row_leader(int I, int& row) const {
    const int v = threadIdx.x + I * NT;
    row = v / VPR;
    return v % VPR == 0 && v < NV;
  }
  template <typename D>
  __device__ __forceinline__ void store_split(D* hi, D* lo, int dst_ld) const {
    static_assert(sizeof(E) == 4, "split store takes an fp32 tile");
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v = threadIdx.x + I * NT;
      if (NV % NT == 0 || v < NV) {
        const int row = v / VPR, c0 = (v % VPR) * 4;
        const float* x = reinterpret_cast<const float*>(&r[I]);
        store4_split<D>(hi + row * dst_ld + c0, lo + row * dst_ld + c0, x[0], x[1], x[2], x[3]);
      }
    });
  }
};

// Global -> LDS in one go (load then store).
template <typename E, int ROWS, int COLS, int NT>
__device__ __forceinline__ void copy_in(E* dst, int dst_ld, const E* __restrict__ src, size_t src_ld) {
  TileCopy<E, ROWS, COLS, NT> t;
  t.load(src, src_ld);
  t.store(dst, dst_ld);
}

// LDS -> global.
template <typename E, int ROWS, int COLS, int NT>
__device__ __forceinline__ void copy_out(E* __restrict__ dst, size_t dst_ld, const E* src, int src_ld) {
  constexpr int VPR = COLS * (int)sizeof(E) / 16;
  constexpr int NV = ROWS * VPR;
  for (int v = threadIdx.x; v < NV; v += NT) {
    const int row = v / VPR, cv = v % VPR;
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst + row * dst_ld) + cv * 16) =
        *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src + row * src_ld) + cv * 16);
  }
}

// ---------------------------------------------------------------------------
// channel-wise decay inside a chunk
// ---------------------------------------------------------------------------
// log alpha is read as max(log alpha, -LOG_ALPHA_FLOOR): a token that would keep
// less than e^-16 (about 1.1e-7, fp32 resolution) of a state row keeps e^-16 of
// it.  The comparison is written so that a NaN passes through.  The floor bounds
// every decay factor the chunked kernels form (see group_ref), so none of them
// can overflow whatever the gates; its derivative is 0 below the floor.
constexpr float LOG_ALPHA_FLOOR = 16.f;
constexpr float ALPHA_FLOOR = 1.12535175e-7f;   // e^-16
__device__ __forceinline__ float floor_log_alpha(float x) { return x < -LOG_ALPHA_FLOOR ? -LOG_ALPHA_FLOOR : x; }
__device__ __forceinline__ bool above_floor(float x) { return !(x < -LOG_ALPHA_FLOOR); }

// Decayed products e^{g_r - g_i} (g = in-chunk cumulative log decay, i <= r) are
// factored through reference rows in the middle of 8-token groups, m(R) = 8R + 4:
//   e^{g_r - g_i} = e^{g_r - g_m(R)} * e^{g_m(R) - g_m(C)} * e^{g_m(C) - g_i}
// with R, C the groups of r and i.  The outer factors span at most 4 and 3 tokens
// (at most e^{4 LOG_ALPHA_FLOOR}), the chain factor is at most 1 for C <= R.
constexpr int NGROUP = CH / 8;
constexpr int NGROUP_PAIRS = NGROUP * (NGROUP - 1) / 2;   // pairs C < R
__host__ __device__ constexpr int group_ref(int R) { return 8 * R + 4; }
__host__ __device__ constexpr int pair_index(int R, int C) { return R * (R - 1) / 2 + C; }   // C < R
__device__ __forceinline__ int pair_r(int pi) {
  int R = 1;
  while ((R + 1) * R / 2 <= pi) ++R;
  return R;
}
__device__ __forceinline__ int pair_c(int pi) { const int R = pair_r(pi); return pi - R * (R - 1) / 2; }
// The outer factors can exceed 1 (the row factor up to e^{4 LOG_ALPHA_FLOOR}, the column
// factor up to e^{3 LOG_ALPHA_FLOOR}), so a chain factor below fp32's normal range can
// belong to a product that is not small.  Column operands whose chain factor falls
// below CHAIN_MIN are therefore formed as one exponential of the summed exponent,
// k_i e^{g_m(R) - g_i} <= 1, which leaves at most one factor above 1 in any product:
// whatever then falls out of fp32 range was below e^-23 of the result.
constexpr float CHAIN_MIN = 1.8e-35f;   // e^-80

// The usual path keeps one reference row in the middle of each 16-row block
// (m = 16a + 8): its row factors span up to 8 tokens and its column factors 7.
// While every such span decays by less than e^-STEEP_SPAN, a product's factors above 1
// stay below e^{2 STEEP_SPAN} = e^64 together, so whatever falls out of fp32 range
// was below e^-23 of the result.  steep_block: does thread (channel tid % dk, block
// tid / dk < 4) see a span at or past that limit in the cumulated log decay g?
constexpr float STEEP_SPAN = 32.f;
__device__ __forceinline__ bool steep_block(const float* g, int ldg, int tid, int dk) {
  const int c = tid % dk, a = tid / dk;
  if (a >= CH / 16) return false;
  const float g0 = g[(16 * a) * ldg + c], gm = g[(16 * a + 8) * ldg + c], g1 = g[(16 * a + 15) * ldg + c];
  return g0 - gm >= STEEP_SPAN || gm - g1 >= STEEP_SPAN;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
// Fused input preparation (kda.h: KDA_FLAG_QK_L2NORM, KDA_FLAG_GATE_LOGSIGMOID).
constexpr float L2N_EPS = 1e-6f;
__device__ __forceinline__ float logsigmoid(float x) { return fminf(x, 0.f) - log1pf(__expf(-fabsf(x))); }
__device__ __forceinline__ float sigmoid_neg(float x) { return 1.f / (1.f + __expf(x)); }   // sigmoid(-x)
template <typename E> __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d) {
  if constexpr (sizeof(E) == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  } else {
    typedef E v4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<v4*>(p) = v4{(E)a, (E)b, (E)c, (E)d};
  }
}
template <typename E> __device__ __forceinline__ void load4(const E* p, float (&x)[4]) {
  if constexpr (sizeof(E) == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  } else {
    typedef E v4 __attribute__((ext_vector_type(4)));
    const v4 v = *reinterpret_cast<const v4*>(p);
    x[0] = (float)v[0]; x[1] = (float)v[1]; x[2] = (float)v[2]; x[3] = (float)v[3];
  }
}
// 8 consecutive elements from global memory as floats (zero when !valid).
template <typename E> __device__ __forceinline__ void load8(const E* p, bool valid, float (&x)[8]) {
  if constexpr (sizeof(E) == 2) {
    typedef E v8 __attribute__((ext_vector_type(8)));
    v8 v = {};
    if (valid) v = *reinterpret_cast<const v8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
  } else {
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      a = *reinterpret_cast<const f32x4*>(p);
      b = *reinterpret_cast<const f32x4*>(p + 4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[j + 4] = b[j]; }
  }
}

// Map a flat block id to (unit, slice) so that all value slices of a unit sit on
// the same XCD (block ids are dealt to the 8 XCDs round robin) and share its L2.
__device__ __forceinline__ bool xcd_unit(int bid, int nsl, int nunits, int& unit, int& slice) {
  const int xcd = bid & 7, idx = bid >> 3;
  slice = idx % nsl;
  unit = (idx / nsl) * 8 + xcd;
  return unit < nunits;
}

// ---------------------------------------------------------------------------
// workspace layout shared by the host planner and the kernels
// ---------------------------------------------------------------------------
// Per (chunk, head) blocks, chunk-major so one head's chunks are strided by H.
// Element counts per block; OP = OpOf<E>::T unless another type is given.
template <typename E, int DK, int DV>
struct WsBlock {
  static constexpr size_t W = (size_t)CH * DK;     // W   [CH][DK]   OP
  static constexpr size_t KHT = (size_t)DK * CH;   // Kh^T[DK][CH]   OP
  static constexpr size_t QT = (size_t)CH * DK;    // Qt  [CH][DK]   OP
  static constexpr size_t UT = (size_t)DV * CH;    // U~^T[DV][CH]   OP
  static constexpr size_t AQK = (size_t)CH * CH;   // Aqk [CH][CH]   OP
  static constexpr size_t TT = (size_t)CH * CH;    // T   [CH][CH]   OP (backward only)
  static constexpr size_t GAM = DK;                // Gamma_C [DK]   float
  // backward only
  static constexpr size_t UTF = (size_t)DV * CH;   // U~^T [DV][CH]   float
  static constexpr size_t G = (size_t)CH * CH;     // un-beta strict Gram [CH][CH]   float
  static constexpr size_t KHF = (size_t)CH * DK;   // Kh  [CH][DK]   float-sized slot: fp32 Kh, or (split
                                                   // types) fp16 hi [CH][DK] followed by fp16 lo [CH][DK]
  static constexpr size_t S = (size_t)DK * DV;     // state entering a chunk [DK][DV]   float
  static constexpr size_t U = (size_t)DV * CH;     // U [CH][DV]   float
  static constexpr size_t DS = (size_t)DK * DV;    // dS' [DK][DV]   float
  static constexpr size_t DU = (size_t)DV * CH;    // dU [CH][DV]  float
};

}  // namespace kda
