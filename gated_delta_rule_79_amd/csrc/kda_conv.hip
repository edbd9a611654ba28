// kda_conv.hip -- short causal convolution with a carried state, on gfx950.
//
// fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier scale", section on
// disaggregated prefill and decode: what a KDA layer hands from one serving
// pool to the next is its recurrent state and its convolution state.  The page
// defines neither.  The reading implemented here: a causal depthwise
// convolution of width W along time over each channel, whose state is the
// sequence's last W - 1 inputs,
//
//     z[t, c] = bias[c] + sum_{j<W} weight[c, j] * X[t - (W-1) + j, c],
//     y = z  or  y = z * sigmoid(z)  (SiLU),
//
// where X is the sequence's input preceded by its W - 1 state rows (zero
// without a state) and the final state is the last W - 1 rows of that
// extended input.  The backward returns the gradients of
// <dy, y> + <d_final_state, final_state> with respect to x, weight, bias and
// the initial state.
//
// The work is elementwise along channels and a W-tap sliding window along
// time, so it is bound by HBM traffic: each thread owns a group of adjacent
// channels (four: one 16-byte fp32 store, or one 8-byte bf16 load, of a token
// row), walks a run of tokens and keeps the window in registers; every load
// and store instruction of a wave covers one contiguous span of a token row,
// so no cache line is written in parts.  Per-tile partial sums of the weight
// and bias gradients are reduced in a fixed order by a second kernel, so the
// results are bitwise reproducible.
#include "kda.h"
#include "kda_internal.hpp"
#include "kda_conv.hpp"

namespace kda {

namespace {

#ifndef KDA_CONV_TT
#define KDA_CONV_TT 64       // forward: tokens per tile
#endif
#ifndef KDA_CONV_U
#define KDA_CONV_U 8         // forward: token rows loaded ahead of their use
#endif
#ifndef KDA_CONV_BWD_U
#define KDA_CONV_BWD_U 4     // backward: token rows (of x and dy) loaded ahead of their use
#endif
constexpr int CV_NT = 256;   // threads per work-group (4 waves)
constexpr int CV_TT = KDA_CONV_TT;
constexpr int CV_U = KDA_CONV_U;
constexpr int CV_UB = KDA_CONV_BWD_U;

// NC consecutive elements as floats.
template <typename E, int NC> __device__ __forceinline__ void cload(const E* p, float (&x)[NC]) {
  if constexpr (sizeof(E) == 2) {
    typedef E vN __attribute__((ext_vector_type(NC)));
    const vN v = *reinterpret_cast<const vN*>(p);
#pragma unroll
    for (int i = 0; i < NC; ++i) x[i] = (float)v[i];
  } else {
#pragma unroll
    for (int i = 0; i < NC; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
      x[i] = v[0]; x[i + 1] = v[1]; x[i + 2] = v[2]; x[i + 3] = v[3];
    }
  }
}

template <typename O, int NC> __device__ __forceinline__ void cstore(O* p, const float (&x)[NC]) {
  if constexpr (sizeof(O) == 2) {
    typedef O vN __attribute__((ext_vector_type(NC)));
    vN v;
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = cvt<O>(x[i]);
    __builtin_nontemporal_store(v, reinterpret_cast<vN*>(p));
  } else {
#pragma unroll
    for (int i = 0; i < NC; i += 4)
      __builtin_nontemporal_store(f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]}, reinterpret_cast<f32x4*>(p + i));
  }
}

template <int NC> __device__ __forceinline__ void czero(float (&x)[NC]) {
#pragma unroll
  for (int i = 0; i < NC; ++i) x[i] = 0.f;
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + __expf(-z)); }
__device__ __forceinline__ float silu_grad(float z) {
  const float s = 1.f / (1.f + __expf(-z));
  return s * (1.f + z * (1.f - s));
}

// Token bounds [a, e) of sequence n.
__device__ __forceinline__ void seq_bounds(const ConvArgs& c, int n, int& a, int& e) {
  if (c.cu) {
    a = c.cu[n];
    e = c.cu[n + 1];
  } else {
    a = n * c.T;
    e = a + c.T;
  }
}

// The sequence holding packed token t (never an empty one): the smallest n
// with cu[n + 1] > t.
__device__ __forceinline__ int seq_of(const ConvArgs& c, int t) {
  if (!c.cu) return t / c.T;
  int lo = 0, hi = c.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (c.cu[mid + 1] <= t) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Extended-input row p of sequence n (starting at token a): a token row when
// p >= a, else state row p - a + W - 1 (zero without a state).
template <typename E, int W, int NC>
__device__ __forceinline__ void ext_row(const ConvArgs& c, int n, int a, int p, int ch, float (&x)[NC]) {
  if (p >= a) cload<E, NC>(static_cast<const E*>(c.x) + (size_t)p * c.D + ch, x);
  else if (c.init) cload<float, NC>(c.init + ((size_t)n * (W - 1) + (p - a + W - 1)) * c.D + ch, x);
  else czero(x);
}

template <int W, int NC>
__device__ __forceinline__ void load_taps(const ConvArgs& c, int ch, float (&w)[W][NC], float (&bias)[NC]) {
#pragma unroll
  for (int i = 0; i < NC; ++i) {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][i] = c.weight[(size_t)(ch + i) * W + j];
    bias[i] = c.bias ? c.bias[ch + i] : 0.f;
  }
}

// Pre-activation of the token whose row is x, after the W - 1 window rows.
template <int W, int NC>
__device__ __forceinline__ void pre_act(const float (&w)[W][NC], const float (&bias)[NC], const float (&win)[W - 1][NC],
                                        const float (&x)[NC], float (&z)[NC]) {
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float s = fmaf(w[W - 1][i], x[i], bias[i]);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) s = fmaf(w[j][i], win[j][i], s);
    z[i] = s;
  }
}

template <int R, int NC> __device__ __forceinline__ void push(float (&win)[R][NC], const float (&x)[NC]) {
#pragma unroll
  for (int j = 0; j < R - 1; ++j)
#pragma unroll
    for (int i = 0; i < NC; ++i) win[j][i] = win[j + 1][i];
#pragma unroll
  for (int i = 0; i < NC; ++i) win[R - 1][i] = x[i];
}

}  // namespace

// ---------------------------------------------------------------------------
// forward: grid (token tiles of CV_TT, XCD-grouped; channel groups / CV_NT)
// ---------------------------------------------------------------------------
template <typename E, typename O, int W>
__global__ __launch_bounds__(CV_NT) void kda_conv_fwd_k(const ConvArgs c) {
  constexpr int NC = 4;
  const int ch = (blockIdx.y * CV_NT + threadIdx.x) * NC;
  if (ch >= c.D) return;
  // Work-group ids are dealt to the 8 XCDs round robin; give each XCD a
  // contiguous run of tiles so a tile's window rows (the previous tile's
  // last W - 1 rows) are found in that XCD's L2.
  const int Tt = c.tokens;
  const int per = ((Tt + CV_TT - 1) / CV_TT + 7) / 8;
  const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int t0 = tile * CV_TT, t1 = min(t0 + CV_TT, Tt);
  if (t0 >= Tt) return;
  float w[W][NC], bias[NC];
  load_taps<W, NC>(c, ch, w, bias);
  const E* x = static_cast<const E*>(c.x);
  O* y = static_cast<O*>(c.y);
  int t = t0;
  while (t < t1) {   // one pass per sequence the tile touches
    const int n = seq_of(c, t);
    int a, e;
    seq_bounds(c, n, a, e);
    const int s1 = min(t1, e);
    float win[W - 1][NC];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) ext_row<E, W, NC>(c, n, a, t - (W - 1) + j, ch, win[j]);
    for (; t < s1; t += CV_U) {
      float xr[CV_U][NC];
#pragma unroll
      for (int u = 0; u < CV_U; ++u)
        if (t + u < s1) cload<E, NC>(x + (size_t)(t + u) * c.D + ch, xr[u]);
#pragma unroll
      for (int u = 0; u < CV_U; ++u) {
        if (t + u < s1) {
          float z[NC];
          pre_act<W, NC>(w, bias, win, xr[u], z);
          if (c.silu) {
#pragma unroll
            for (int i = 0; i < NC; ++i) z[i] = silu(z[i]);
          }
          cstore<O, NC>(y + (size_t)(t + u) * c.D + ch, z);
          push<W - 1, NC>(win, xr[u]);
        }
      }
    }
    t = s1;
  }
}

// Final state: the last W - 1 extended rows of each sequence.  Grid (channel
// groups / CV_NT, N).  Every source row is read before any row is written, so
// final_state may alias init_state.
template <typename E, int W>
__global__ __launch_bounds__(CV_NT) void kda_conv_final_k(const ConvArgs c) {
  constexpr int NC = 4;
  const int ch = (blockIdx.x * CV_NT + threadIdx.x) * NC;
  if (ch >= c.D) return;
  const int n = blockIdx.y;
  int a, e;
  seq_bounds(c, n, a, e);
  float r[W - 1][NC];
#pragma unroll
  for (int i = 0; i < W - 1; ++i) ext_row<E, W, NC>(c, n, a, e - (W - 1) + i, ch, r[i]);
#pragma unroll
  for (int i = 0; i < W - 1; ++i) cstore<float, NC>(c.final_state + ((size_t)n * (W - 1) + i) * c.D + ch, r[i]);
}

// ---------------------------------------------------------------------------
// backward: grid (token tiles of CONV_BWD_TILE; channel groups / CV_NT)
// ---------------------------------------------------------------------------
// For each token p of the tile (and W - 1 tokens past it, inside the same
// sequence) the thread recomputes z[p] from its window, forms dz = dy *
// act'(z), accumulates dweight[j] += dz * X[p - (W-1) + j] and dbias += dz for
// the tile's own tokens, and emits dx[p - (W-1)] = sum_j weight[j] dz[p - j]
// (plus the final-state gradient for the sequence's last W - 1 tokens) once
// its last contributing dz is known.  Tokens past the sequence end contribute
// dz = 0.
template <typename E, typename O, int W>
__global__ __launch_bounds__(CV_NT) void kda_conv_bwd_k(const ConvArgs c) {
  constexpr int NC = 4;
  const int ch = (blockIdx.y * CV_NT + threadIdx.x) * NC;
  if (ch >= c.D) return;
  const int Tt = c.tokens;
  const int tile = blockIdx.x;
  const int t0 = tile * CONV_BWD_TILE, t1 = min(t0 + CONV_BWD_TILE, Tt);
  float w[W][NC], bias[NC];
  load_taps<W, NC>(c, ch, w, bias);
  float dw[W][NC], db[NC];
#pragma unroll
  for (int j = 0; j < W; ++j) czero(dw[j]);
  czero(db);
  const E* x = static_cast<const E*>(c.x);
  const E* dy = static_cast<const E*>(c.dy);
  O* dx = static_cast<O*>(c.dx);
  int t = t0;
  while (t < t1) {
    const int n = seq_of(c, t);
    int a, e;
    seq_bounds(c, n, a, e);
    const int s0 = t, s1 = min(t1, e), send = s1 + W - 1;
    float xwin[W - 1][NC], dzw[W - 1][NC];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      ext_row<E, W, NC>(c, n, a, s0 - (W - 1) + j, ch, xwin[j]);
      czero(dzw[j]);   // dz before s0 only reaches dx rows before s0, which this pass does not emit
    }
    for (int p0 = s0; p0 < send; p0 += CV_UB) {
      float xr[CV_UB][NC], gr[CV_UB][NC];
#pragma unroll
      for (int u = 0; u < CV_UB; ++u) {
        const int p = p0 + u;
        if (p < send && p < e) {
          cload<E, NC>(x + (size_t)p * c.D + ch, xr[u]);
          cload<E, NC>(dy + (size_t)p * c.D + ch, gr[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < CV_UB; ++u) {
        const int p = p0 + u;
        if (p < send) {
          float dz[NC];
          if (p < e) {
            float z[NC];
            pre_act<W, NC>(w, bias, xwin, xr[u], z);
#pragma unroll
            for (int i = 0; i < NC; ++i) dz[i] = c.silu ? gr[u][i] * silu_grad(z[i]) : gr[u][i];
            if (p < s1) {
#pragma unroll
              for (int i = 0; i < NC; ++i) {
#pragma unroll
                for (int j = 0; j < W - 1; ++j) dw[j][i] = fmaf(dz[i], xwin[j][i], dw[j][i]);
                dw[W - 1][i] = fmaf(dz[i], xr[u][i], dw[W - 1][i]);
                db[i] += dz[i];
              }
            }
            push<W - 1, NC>(xwin, xr[u]);
          } else {
            czero(dz);
          }
          const int tq = p - (W - 1);   // token whose dx is now complete
          if (tq >= s0) {
            float g[NC];
#pragma unroll
            for (int i = 0; i < NC; ++i) {
              float s = w[0][i] * dz[i];
#pragma unroll
              for (int j = 1; j < W; ++j) s = fmaf(w[j][i], dzw[W - 1 - j][i], s);
              g[i] = s;
            }
            if (c.dfinal && tq >= e - (W - 1)) {
              float f[NC];
              cload<float, NC>(c.dfinal + ((size_t)n * (W - 1) + (tq - e + W - 1)) * c.D + ch, f);
#pragma unroll
              for (int i = 0; i < NC; ++i) g[i] += f[i];
            }
            cstore<O, NC>(dx + (size_t)tq * c.D + ch, g);
          }
          push<W - 1, NC>(dzw, dz);
        }
      }
    }
    t = s1;
  }
  // per-tile partial sums: part[tile][j][D], j = 0..W-1 weight taps, W = bias
#pragma unroll
  for (int j = 0; j < W; ++j) cstore<float, NC>(c.part + ((size_t)tile * (W + 1) + j) * c.D + ch, dw[j]);
  cstore<float, NC>(c.part + ((size_t)tile * (W + 1) + W) * c.D + ch, db);
}

// Initial-state gradient: rows r < W - 1 of the extended-input gradient,
// sum_j weight[j] dz[r - j] over the sequence's first tokens, plus the
// final-state gradient where the sequence is shorter than the state.  Grid
// (channel groups / CV_NT, N).
template <typename E, int W>
__global__ __launch_bounds__(CV_NT) void kda_conv_dinit_k(const ConvArgs c) {
  constexpr int NC = 4;
  const int ch = (blockIdx.x * CV_NT + threadIdx.x) * NC;
  if (ch >= c.D) return;
  const int n = blockIdx.y;
  int a, e;
  seq_bounds(c, n, a, e);
  const int m = min(e - a, W - 1);   // tokens whose dz reach a state row
  float w[W][NC], bias[NC];
  load_taps<W, NC>(c, ch, w, bias);
  float win[W - 1][NC], dz[W - 1][NC];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    ext_row<E, W, NC>(c, n, a, a - (W - 1) + j, ch, win[j]);
    czero(dz[j]);
  }
#pragma unroll
  for (int p = 0; p < W - 1; ++p) {
    if (p < m) {
      float xr[NC], gr[NC], z[NC];
      cload<E, NC>(static_cast<const E*>(c.x) + (size_t)(a + p) * c.D + ch, xr);
      cload<E, NC>(static_cast<const E*>(c.dy) + (size_t)(a + p) * c.D + ch, gr);
      pre_act<W, NC>(w, bias, win, xr, z);
#pragma unroll
      for (int i = 0; i < NC; ++i) dz[p][i] = c.silu ? gr[i] * silu_grad(z[i]) : gr[i];
      push<W - 1, NC>(win, xr);
    }
  }
  const int L = e - a;
#pragma unroll
  for (int r = 0; r < W - 1; ++r) {
    float g[NC];
    czero(g);
#pragma unroll
    for (int j = 0; j <= r; ++j)
      if (r - j < m) {
#pragma unroll
        for (int i = 0; i < NC; ++i) g[i] = fmaf(w[j][i], dz[r - j][i], g[i]);
      }
    if (c.dfinal && r >= L) {
      float f[NC];
      cload<float, NC>(c.dfinal + ((size_t)n * (W - 1) + (r - L)) * c.D + ch, f);
#pragma unroll
      for (int i = 0; i < NC; ++i) g[i] += f[i];
    }
    cstore<float, NC>(c.dinit + ((size_t)n * (W - 1) + r) * c.D + ch, g);
  }
}

// dweight [D][W] and dbias [D]: the tiles' partial sums added in a fixed
// order.  A work-group takes 64 adjacent partial-sum columns (column = tap or
// bias row j times D plus channel) and its four waves take every fourth tile
// each; the four stripe sums are then added in stripe order.
constexpr int CV_RED_COLS = 64;
template <int W>
__global__ __launch_bounds__(CV_NT) void kda_conv_reduce_k(const ConvArgs c, int tiles) {
  __shared__ float part[CV_NT / CV_RED_COLS][CV_RED_COLS];
  const int ncol = (W + 1) * c.D;
  const int l = threadIdx.x % CV_RED_COLS, stripe = threadIdx.x / CV_RED_COLS;
  const int col = blockIdx.x * CV_RED_COLS + l;
  constexpr int NS = CV_NT / CV_RED_COLS;
  float s = 0.f;
  if (col < ncol) {
    const float* p = c.part + col;
    int t = stripe;
    for (; t + 3 * NS < tiles; t += 4 * NS) {   // four tiles in flight, added in order
      const float a = p[(size_t)t * ncol], b = p[(size_t)(t + NS) * ncol];
      const float d = p[(size_t)(t + 2 * NS) * ncol], e = p[(size_t)(t + 3 * NS) * ncol];
      s += a;
      s += b;
      s += d;
      s += e;
    }
    for (; t < tiles; t += NS) s += p[(size_t)t * ncol];
  }
  part[stripe][l] = s;
  __syncthreads();
  if (stripe == 0 && col < ncol) {
    float r = part[0][l];
#pragma unroll
    for (int k = 1; k < NS; ++k) r += part[k][l];
    const int j = col / c.D, ch = col % c.D;
    if (j < W) c.dweight[(size_t)ch * W + j] = r;
    else if (c.dbias) c.dbias[ch] = r;
  }
}

// ---------------------------------------------------------------------------
// decode / replay: grid (channel groups / CV_NT, B)
// ---------------------------------------------------------------------------
template <typename E, typename O, int W>
__global__ __launch_bounds__(CV_NT) void kda_conv_decode_k(const ConvArgs c) {
  constexpr int NC = 4;
  const int ch = (blockIdx.x * CV_NT + threadIdx.x) * NC;
  if (ch >= c.D) return;
  const int b = blockIdx.y, T = c.T;
  const int slot = c.idx ? c.idx[b] : b;
  O* y = static_cast<O*>(c.y);
  if (slot < 0 || slot >= c.pool_size) {   // padding entry: zero outputs, no state touched
    float zero[NC];
    czero(zero);
    for (int u = 0; u < T; ++u) cstore<O, NC>(y + ((size_t)b * T + u) * c.D + ch, zero);
    return;
  }
  const int ncom = c.ncommit ? min(max(c.ncommit[b], 0), T) : T;
  float w[W][NC], bias[NC];
  load_taps<W, NC>(c, ch, w, bias);
  float* st = c.pool + (size_t)slot * (W - 1) * c.D + ch;
  float win[W - 1][NC], keep[W - 1][NC];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    cload<float, NC>(st + (size_t)j * c.D, win[j]);
#pragma unroll
    for (int i = 0; i < NC; ++i) keep[j][i] = win[j][i];
  }
  const E* x = static_cast<const E*>(c.x);
  for (int u = 0; u < T; ++u) {
    float xr[NC], z[NC];
    cload<E, NC>(x + ((size_t)b * T + u) * c.D + ch, xr);
    pre_act<W, NC>(w, bias, win, xr, z);
    if (c.silu) {
#pragma unroll
      for (int i = 0; i < NC; ++i) z[i] = silu(z[i]);
    }
    cstore<O, NC>(y + ((size_t)b * T + u) * c.D + ch, z);
    push<W - 1, NC>(win, xr);
    if (u + 1 == ncom) {
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int i = 0; i < NC; ++i) keep[j][i] = win[j][i];
    }
  }
  if (ncom > 0) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) cstore<float, NC>(st + (size_t)j * c.D, keep[j]);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {
inline unsigned cgroups(int D, int nc) { return (unsigned)((D / nc + CV_NT - 1) / CV_NT); }
}  // namespace

template <typename E, typename O, int W> hipError_t launch_conv_fwd(const ConvArgs& c, hipStream_t st) {
  if (c.tokens > 0)
    KDA_TIMED("kda_conv_fwd", st,
              hipLaunchKernelGGL((kda_conv_fwd_k<E, O, W>), dim3(((c.tokens + CV_TT - 1) / CV_TT + 7) / 8 * 8, cgroups(c.D, 4)),
                                 dim3(CV_NT), 0, st, c));
  if (c.final_state)
    KDA_TIMED("kda_conv_final", st,
              hipLaunchKernelGGL((kda_conv_final_k<E, W>), dim3(cgroups(c.D, 4), c.N), dim3(CV_NT), 0, st, c));
  return hipGetLastError();
}

template <typename E, typename O, int W> hipError_t launch_conv_bwd(const ConvArgs& c, hipStream_t st) {
  const int tiles = (c.tokens + CONV_BWD_TILE - 1) / CONV_BWD_TILE;
  if (tiles > 0)
    KDA_TIMED("kda_conv_bwd", st,
              hipLaunchKernelGGL((kda_conv_bwd_k<E, O, W>), dim3(tiles, cgroups(c.D, 4)), dim3(CV_NT), 0, st, c));
  KDA_TIMED("kda_conv_reduce", st,
            hipLaunchKernelGGL((kda_conv_reduce_k<W>), dim3(((W + 1) * c.D + CV_RED_COLS - 1) / CV_RED_COLS),
                               dim3(CV_NT), 0, st, c, tiles));
  if (c.dinit)
    KDA_TIMED("kda_conv_dinit", st,
              hipLaunchKernelGGL((kda_conv_dinit_k<E, W>), dim3(cgroups(c.D, 4), c.N), dim3(CV_NT), 0, st, c));
  return hipGetLastError();
}

template <typename E, typename O, int W> hipError_t launch_conv_decode(const ConvArgs& c, hipStream_t st) {
  KDA_TIMED("kda_conv_decode", st,
            hipLaunchKernelGGL((kda_conv_decode_k<E, O, W>), dim3(cgroups(c.D, 4), c.B), dim3(CV_NT), 0, st, c));
  return hipGetLastError();
}

#define KDA_CONV_INST(E, O, W)                                                          \
  template hipError_t launch_conv_fwd<E, O, W>(const ConvArgs&, hipStream_t);           \
  template hipError_t launch_conv_bwd<E, O, W>(const ConvArgs&, hipStream_t);           \
  template hipError_t launch_conv_decode<E, O, W>(const ConvArgs&, hipStream_t);
#define KDA_CONV_INST_W(E, O) KDA_CONV_INST(E, O, 2) KDA_CONV_INST(E, O, 3) KDA_CONV_INST(E, O, 4)
KDA_CONV_INST_W(float, float)
KDA_CONV_INST_W(bf16, float)
KDA_CONV_INST_W(bf16, bf16)
#undef KDA_CONV_INST_W
#undef KDA_CONV_INST

}  // namespace kda
