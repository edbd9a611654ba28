// kda_fwd.hip -- forward pass of Kimi Delta Attention on gfx950.
//
// The method (fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier scale",
// section on Kimi Delta Attention) updates a per-head state S (dk x dv) with
// channel-wise gating; the page says fast training must run the chunk-local
// work in parallel and keep the recurrent dependency and the traffic of
// intermediates small.  Per chunk of C = 64 tokens (state S entering it,
// g = in-chunk cumulative sum of log_alpha, Gamma = exp(g)):
//
//   K+ = K*Gamma, K- = K/Gamma, Qt = Q*Gamma, Kh = K*exp(g_C - g)
//   A   = strict_tril(diag(beta) K+ K-^T)       T = (I + A)^-1
//   W   = T diag(beta) K+                       U~ = T diag(beta) V
//   U   = U~ - W S
//   O   = scale * (Qt S + tril(Qt K-^T) U)
//   S'  = diag(Gamma_C) S + Kh^T U
//
// which is the token recurrence S_t = (I - b k k^T) Diag(a) S + b k v^T,
// o_t = scale S_t^T q_t summed in closed form over the chunk (the rows of the
// unit-lower-triangular system (I + A) U = ... are the per-token delta steps).
//
// Kernels:
//   kda_chunk_map   : (sequence, chunk) table from cu_seqlens on the device.
//   kda_prep        : chunk-parallel; cumsum, decayed Gram blocks, T by
//                     blocked forward substitution, W and U~ on MFMA.
//   kda_state       : sequential over the chunks of one (sequence, head,
//                     value-column slice); S stays in registers, output fused.
//
// The decayed Gram blocks never form K- = K/Gamma: block (a, b) of rows a and
// columns b uses a reference row m in the middle of row block a and factors
// exp(g_r - g_i) = exp(g_r - g_m) * exp(g_m - g_i), so no factor exceeds the
// decay of 8 consecutive tokens.
#include "kda_internal.hpp"

namespace kda {

// ---------------------------------------------------------------------------
// chunk map
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kda_chunk_map(const int32_t* __restrict__ cu, int N, int T,
                                                     ChunkInfo* __restrict__ chunks,
                                                     int32_t* __restrict__ seq_chunk0, int max_chunks) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int s0 = tid * per, s1 = min(N, s0 + per);
  // cu_seqlens contents are a caller precondition; clamping keeps every later
  // index in bounds even when they are wrong (results are then meaningless)
  const int ntok = cu ? T : N * T;
  auto seq_start = [&](int s) -> int { return cu ? min(max(cu[s], 0), ntok) : s * T; };
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (max(seq_start(s + 1) - seq_start(s), 0) + CH - 1) / CH;
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int run = part[tid] - local;
  for (int s = s0; s < s1; ++s) {
    seq_chunk0[s] = min(run, max_chunks);
    run += (max(seq_start(s + 1) - seq_start(s), 0) + CH - 1) / CH;
  }
  if (tid == 1023) seq_chunk0[N] = min(part[1023], max_chunks);
  __threadfence();
  __syncthreads();
  const volatile int32_t* sc0 = seq_chunk0;  // written above by other threads of this block
  const int total = sc0[N];
  for (int j = tid; j < max_chunks; j += 1024) {
    ChunkInfo ci{0, 0, 0, 0};
    if (j < total) {
      int lo = 0, hi = N;  // last s with seq_chunk0[s] <= j
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sc0[mid] <= j) lo = mid; else hi = mid;
      }
      const int st = seq_start(lo), en = seq_start(lo + 1);
      const int idx = j - sc0[lo];
      ci.seq = lo;
      ci.idx = idx;
      ci.t0 = st + idx * CH;
      ci.len = max(0, min(CH, en - ci.t0));
    }
    chunks[j] = ci;
  }
}

hipError_t launch_chunk_map(const Args& a, hipStream_t st) {
  hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(1024), 0, st, a.cu, a.N, a.T, a.chunks, a.seq_chunk0,
                     a.max_chunks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
template <typename E> __device__ __forceinline__ void store4(E* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 o = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
template <typename E> __device__ __forceinline__ void load4(const E* p, float (&x)[4]);
template <> __device__ __forceinline__ void load4<bf16>(const bf16* p, float (&x)[4]) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  x[0] = (float)v[0]; x[1] = (float)v[1]; x[2] = (float)v[2]; x[3] = (float)v[3];
}
template <> __device__ __forceinline__ void load4<float>(const float* p, float (&x)[4]) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
}
// 8 consecutive elements from global memory as floats (zero when !valid).
template <typename E> __device__ __forceinline__ void load8(const E* p, bool valid, float (&x)[8]) {
  if constexpr (sizeof(E) == 2) {
    bf16x8 v = {};
    if (valid) v = *reinterpret_cast<const bf16x8*>(p);
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

// ---------------------------------------------------------------------------
// prep: chunk-parallel part
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
struct PrepLds {
  static constexpr int P = PADE<E>;
  static constexpr int LDG = DK + 4;   // float g[CH][LDG]
  static constexpr int LDK = DK + P;   // E k[CH][LDK]
  static constexpr int LDT = CH + P;   // E x[*][LDT]
  static constexpr int LDA = CH + 4;   // float A[CH][LDA]
  static constexpr size_t G = 0;
  static constexpr size_t K = G + (size_t)CH * LDG * 4;
  static constexpr size_t KPT = K + (size_t)CH * LDK * sizeof(E);
  static constexpr size_t VT = KPT + (size_t)DK * LDT * sizeof(E);
  static constexpr size_t A = VT + (size_t)DV * LDT * sizeof(E);
  static constexpr size_t TOT = A + (size_t)CH * LDA * 4;
  static constexpr size_t BETA = TOT + 4 * DK * 4;
  static constexpr size_t X = BETA + CH * 4;
  static constexpr size_t BYTES = X + 3 * 256 * 4;
  // aliases used once the Gram blocks are done
  static constexpr size_t T = G;     // float [CH][LDA]  (fits in g)
  static constexpr size_t TE = K;    // E [CH][LDT]      (fits in k)
  static_assert((size_t)CH * LDA * 4 <= (size_t)CH * LDG * 4, "T alias");
  static_assert((size_t)CH * LDT * sizeof(E) <= (size_t)CH * LDK * sizeof(E), "Te alias");
  static_assert(BYTES <= 163840, "prep LDS");
};

template <typename E, int DK, int DV, bool BWD>
__global__ __launch_bounds__(256) void kda_prep(const Args a) {
  using L = PrepLds<E, DK, DV>;
  constexpr int NT = 256;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int j = blockIdx.x, h = blockIdx.y, H = a.H;
  const ChunkInfo ci = a.chunks[j];
  if (ci.len <= 0) return;
  const int len = ci.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;

  float* sG = reinterpret_cast<float*>(smem + L::G);
  E* sK = reinterpret_cast<E*>(smem + L::K);
  E* sKpT = reinterpret_cast<E*>(smem + L::KPT);
  E* sVT = reinterpret_cast<E*>(smem + L::VT);
  float* sA = reinterpret_cast<float*>(smem + L::A);
  float* sTot = reinterpret_cast<float*>(smem + L::TOT);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sX = reinterpret_cast<float*>(smem + L::X);

  const size_t rk = (size_t)H * DK, rv = (size_t)H * DV;  // token strides
  const E* qh = reinterpret_cast<const E*>(a.q) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* kh = reinterpret_cast<const E*>(a.k) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* lh = reinterpret_cast<const E*>(a.la) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* vh = reinterpret_cast<const E*>(a.v) + (size_t)ci.t0 * rv + (size_t)h * DV;
  const E* bh = reinterpret_cast<const E*>(a.beta) + (size_t)ci.t0 * H + h;

  using WB = WsBlock<E, DK, DV>;
  const size_t blk = (size_t)j * H + h;
  E* wW = reinterpret_cast<E*>(a.wsW) + blk * WB::W;
  float* wKhT = reinterpret_cast<float*>(a.wsKhT) + blk * WB::KHT;
  E* wQt = reinterpret_cast<E*>(a.wsQt) + blk * WB::QT;
  float* wUt = reinterpret_cast<float*>(a.wsUt) + blk * WB::UT;
  float* wAqk = reinterpret_cast<float*>(a.wsAqk) + blk * WB::AQK;
  float* wGam = a.wsGam + blk * WB::GAM;

  // ---- 1. cumulative log-decay g (fp32), k rows, v^T, beta
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    float acc = 0.f;
    for (int r = s * RPS; r < (s + 1) * RPS; ++r) {
      acc += r < len ? f32(lh[r * rk + c]) : 0.f;
      sG[r * L::LDG + c] = acc;
    }
    sTot[s * DK + c] = acc;
  }
  if (tid < CH) sBeta[tid] = tid < len ? f32(bh[(size_t)tid * H]) : 0.f;
  {
    constexpr int EPV = 16 / (int)sizeof(E);
    constexpr int VPR = DK / EPV, NV = CH * VPR;
    for (int v = tid; v < NV; v += NT) {
      const int r = v / VPR, cv = v % VPR;
      uint4 x = {0u, 0u, 0u, 0u};
      if (r < len) x = *reinterpret_cast<const uint4*>(kh + r * rk + cv * EPV);
      *reinterpret_cast<uint4*>(sK + r * L::LDK + cv * EPV) = x;
    }
  }
  {
    constexpr int VPR = DV / 8, NV = CH * VPR;
    for (int v = tid; v < NV; v += NT) {
      const int r = v / VPR, c0 = (v % VPR) * 8;
      float x[8];
      load8<E>(vh + r * rv + c0, r < len, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) sVT[(c0 + i) * L::LDT + r] = cvt<E>(x[i]);
    }
  }
  __syncthreads();
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    if (s > 0) {
      float off = 0.f;
      for (int s2 = 0; s2 < s; ++s2) off += sTot[s2 * DK + c];
      for (int r = s * RPS; r < (s + 1) * RPS; ++r) sG[r * L::LDG + c] += off;
    }
  }
  __syncthreads();

  // ---- 2. elementwise: K+^T (LDS), Kh^T, Qt, Gamma_C (workspace)
  {
    const int r = tid & (CH - 1);
    for (int c = tid / CH; c < DK; c += NT / CH) {
      const float g = sG[r * L::LDG + c];
      const float gl = sG[(CH - 1) * L::LDG + c];
      const float kv = f32(sK[r * L::LDK + c]);
      sKpT[c * L::LDT + r] = cvt<E>(kv * __expf(g));
      wKhT[c * CH + r] = kv * __expf(gl - g);
    }
    constexpr int VPR = DK / 8, NV = CH * VPR;
    for (int v = tid; v < NV; v += NT) {
      const int rr = v / VPR, c0 = (v % VPR) * 8;
      float x[8];
      load8<E>(qh + rr * rk + c0, rr < len, x);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[i] * __expf(sG[rr * L::LDG + c0 + i]);
      store4<E>(wQt + rr * DK + c0, y[0], y[1], y[2], y[3]);
      store4<E>(wQt + rr * DK + c0 + 4, y[4], y[5], y[6], y[7]);
    }
    for (int c = tid; c < DK; c += NT) wGam[c] = __expf(sG[(CH - 1) * L::LDG + c]);
  }

  // ---- 3. decayed Gram blocks: wave w owns row block a = w
  {
    const int ab = w;
    const int ref = 16 * ab + 8;
    const int r = 16 * ab + r16;
    // the gated factors are split operands: their rounding would otherwise
    // dominate the error of the intra-chunk terms
    constexpr int NKS = DK / 32;
    SFrag<E> fk[NKS], fq[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int c0 = 32 * ks + 8 * q4;
      float xq[8], xk[8];
      load8<E>(qh + r * rk + c0, r < len, xq);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __expf(sG[r * L::LDG + c0 + i] - sG[ref * L::LDG + c0 + i]);
        xk[i] = f32(sK[r * L::LDK + c0 + i]) * e;
        xq[i] *= e;
      }
      fk[ks] = sfrag_from<E>(xk);
      fq[ks] = sfrag_from<E>(xq);
    }
    for (int b = 0; b <= ab; ++b) {
      f32x4 akk = zero4(), aqk = zero4();
      const int i = 16 * b + r16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * q4;
        float xr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          xr[u] = f32(sK[i * L::LDK + c0 + u]) * __expf(sG[ref * L::LDG + c0 + u] - sG[i * L::LDG + c0 + u]);
        const SFrag<E> fr = sfrag_from<E>(xr);
        akk = mma_ss(fk[ks], fr, akk);
        aqk = mma_ss(fq[ks], fr, aqk);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * ab + 4 * q4 + ii, cc = 16 * b + r16;
        sA[rr * L::LDA + cc] = cc < rr ? sBeta[rr] * akk[ii] : 0.f;
        wAqk[rr * CH + cc] = cc <= rr ? aqk[ii] : 0.f;
      }
    }
    for (int b = ab + 1; b < 4; ++b) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * ab + 4 * q4 + ii, cc = 16 * b + r16;
        sA[rr * L::LDA + cc] = 0.f;
        wAqk[rr * CH + cc] = 0.f;
      }
    }
  }
  __syncthreads();

  // ---- 4. T = (I + A)^-1 : diagonal 16x16 blocks by substitution, then block rows
  float* sT = reinterpret_cast<float*>(smem + L::T);
  {
    const int ab = w, c = l & 15, s = l >> 4;
    float x[4] = {0.f, 0.f, 0.f, 0.f};  // x[m] = T_aa[s + 4m][c]
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = s + 4 * m;
        if (i < rr) part += sA[(16 * ab + rr) * L::LDA + 16 * ab + i] * x[m];
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const float val = rr == c ? 1.f : (rr > c ? -part : 0.f);
      if (s == (rr & 3)) x[rr >> 2] = val;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) sT[(16 * ab + s + 4 * m) * L::LDA + 16 * ab + c] = x[m];
    for (int b = ab + 1; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 4; ++m) sT[(16 * ab + s + 4 * m) * L::LDA + 16 * b + c] = 0.f;
  }
  __syncthreads();
  for (int d = 1; d < 4; ++d) {
    const int nb = 4 - d;
    for (int o = tid; o < nb * 256; o += NT) {
      const int bl = o >> 8, rr = (o >> 4) & 15, cc = o & 15, ab = bl + d, b = bl;
      float acc = 0.f;
      for (int kk = 16 * b; kk < 16 * ab; ++kk) acc += sA[(16 * ab + rr) * L::LDA + kk] * sT[kk * L::LDA + 16 * b + cc];
      sX[bl * 256 + rr * 16 + cc] = acc;
    }
    __syncthreads();
    for (int o = tid; o < nb * 256; o += NT) {
      const int bl = o >> 8, rr = (o >> 4) & 15, cc = o & 15, ab = bl + d, b = bl;
      float acc = 0.f;
      for (int kk = 0; kk <= rr; ++kk) acc += sT[(16 * ab + rr) * L::LDA + 16 * ab + kk] * sX[bl * 256 + kk * 16 + cc];
      sT[(16 * ab + rr) * L::LDA + 16 * b + cc] = -acc;
    }
    __syncthreads();
  }

  // ---- 5. Te = T diag(beta) in the operand type; W = Te K+, U~ = Te V
  E* sTe = reinterpret_cast<E*>(smem + L::TE);
  for (int o = tid; o < CH * CH; o += NT) {
    const int rr = o / CH, cc = o % CH;
    const float t = sT[rr * L::LDA + cc];
    sTe[rr * L::LDT + cc] = cvt<E>(t * sBeta[cc]);
    if constexpr (BWD) reinterpret_cast<float*>(a.wsT)[blk * WB::TT + o] = t;
  }
  __syncthreads();
  {
    // W^T tiles: C'[ch][tok] = sum_i K+^T[ch][i] Te[tok][i]; lane gets W[tok][4 consecutive ch]
    constexpr int NTI = (CH / 16) * (DK / 16);
    for (int t = w; t < NTI; t += 4) {
      const int mt = t % (CH / 16), nt = t / (CH / 16);
      const f32x4 acc = tile_mm<CH>([&](int rr, int k) { return frag_row<E>(sKpT, L::LDT, 16 * nt + rr, k); },
                                    [&](int rr, int k) { return frag_row<E>(sTe, L::LDT, 16 * mt + rr, k); },
                                    zero4());
      store4<E>(wW + (16 * mt + r16) * DK + 16 * nt + 4 * q4, acc[0], acc[1], acc[2], acc[3]);
    }
    // U~ tiles: C[tok][dv]; lane holds 4 consecutive tokens of one value column -> U~^T rows
    constexpr int NTU = (CH / 16) * (DV / 16);
    for (int t = w; t < NTU; t += 4) {
      const int mt = t % (CH / 16), nt = t / (CH / 16);
      const f32x4 acc = tile_mm<CH>([&](int rr, int k) { return frag_row<E>(sTe, L::LDT, 16 * mt + rr, k); },
                                    [&](int rr, int k) { return frag_row<E>(sVT, L::LDT, 16 * nt + rr, k); },
                                    zero4());
      *reinterpret_cast<f32x4*>(wUt + (16 * nt + r16) * CH + 16 * mt + 4 * q4) = acc;
    }
  }
}


// ---------------------------------------------------------------------------
// sequential state pass (forward outputs, or the per-chunk states for backward)
// ---------------------------------------------------------------------------
// One work-group walks the chunks of one (sequence, head, value slice of DVS
// columns) in order.  Eight waves: waves 0-3 form U = U~ - W S for token tile
// w, waves 4-7 form Qt S and then the output rows of tile w-4; every wave
// updates one or more 16x16 tiles of S.  S stays in fp32 registers; it is
// written to LDS as a split operand for the two products that read it.
template <typename E, int DK, int DV, int DVS, bool OUT>
struct StateLds {
  static constexpr int P = PADE<E>;
  static constexpr int LDK = DK + P;
  static constexpr int LDT = CH + P;
  static constexpr int LDF = CH + 4;
  static constexpr size_t W = 0;                                                 // E     [CH][LDK]
  static constexpr size_t QT = W + (size_t)CH * LDK * sizeof(E);                 // E     [CH][LDK]  (OUT)
  static constexpr size_t KHT = QT + (OUT ? (size_t)CH * LDK * sizeof(E) : 0);   // float [DK][LDF]
  static constexpr size_t AQK = KHT + (size_t)DK * LDF * 4;                      // float [CH][LDF]  (OUT)
  static constexpr size_t UT = AQK + (OUT ? (size_t)CH * LDF * 4 : 0);           // float [DVS][CH]
  static constexpr size_t GAM = UT + (size_t)DVS * CH * 4;                       // float [DK]
  static constexpr size_t STH = GAM + (size_t)DK * 4;                            // E     [DVS][LDK]
  static constexpr size_t STL = STH + (size_t)DVS * LDK * sizeof(E);             // E     [DVS][LDK]
  static constexpr size_t ULH = STL + (size_t)DVS * LDK * sizeof(E);             // E     [DVS][LDT]
  static constexpr size_t ULL = ULH + (size_t)DVS * LDT * sizeof(E);             // E     [DVS][LDT]
  static constexpr size_t BYTES = ULL + (size_t)DVS * LDT * sizeof(E);
  static_assert(BYTES <= 163840, "state LDS");
};

// Map a flat block id to (unit, slice) so that all value slices of a unit sit on
// the same XCD (block ids are dealt to the 8 XCDs round robin) and share its L2.
__device__ __forceinline__ bool xcd_unit(int bid, int nsl, int nunits, int& unit, int& slice) {
  const int xcd = bid & 7, idx = bid >> 3;
  slice = idx % nsl;
  unit = (idx / nsl) * 8 + xcd;
  return unit < nunits;
}

template <typename E, typename O, int DK, int DV, int DVS, bool OUT>
__global__ __launch_bounds__(512) void kda_state(const Args a) {
  using L = StateLds<E, DK, DV, DVS, OUT>;
  using WB = WsBlock<E, DK, DV>;
  constexpr int NT = 512, NSL = DV / DVS;
  constexpr int MTS = DK / 16, NTS = DVS / 16;   // state tiles (channel x column)
  constexpr int NST = MTS * NTS;
  constexpr int SPW = (NST + 7) / 8;             // state tiles per wave (tile t -> wave t % 8)
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  int unit, sl;
  if (!xcd_unit(blockIdx.x, NSL, a.N * a.H, unit, sl)) return;
  const int seq = unit / a.H, h = unit % a.H, H = a.H;
  const int n0 = sl * DVS;
  const int l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  const int c0 = a.seq_chunk0[seq], nch = a.seq_chunk0[seq + 1] - c0;

  E* sW = reinterpret_cast<E*>(smem + L::W);
  E* sQt = reinterpret_cast<E*>(smem + L::QT);
  float* sKhT = reinterpret_cast<float*>(smem + L::KHT);
  float* sAqk = reinterpret_cast<float*>(smem + L::AQK);
  float* sUt = reinterpret_cast<float*>(smem + L::UT);
  float* sGam = reinterpret_cast<float*>(smem + L::GAM);
  E* sSTh = reinterpret_cast<E*>(smem + L::STH);
  E* sSTl = reinterpret_cast<E*>(smem + L::STL);
  E* sULh = reinterpret_cast<E*>(smem + L::ULH);
  E* sULl = reinterpret_cast<E*>(smem + L::ULL);

  // kernel-argument fields are copied to locals so the argument block never
  // has its address taken (that would place it in scratch)
  const E* gW = reinterpret_cast<const E*>(a.wsW);
  const E* gQt = reinterpret_cast<const E*>(a.wsQt);
  const float* gAqk = reinterpret_cast<const float*>(a.wsAqk);
  const float* gKhT = reinterpret_cast<const float*>(a.wsKhT);
  const float* gUt = reinterpret_cast<const float*>(a.wsUt);
  const float* gGam = a.wsGam;
  float* gS = reinterpret_cast<float*>(a.wsS);
  O* gOut = reinterpret_cast<O*>(a.out);
  const ChunkInfo* gChunks = a.chunks;
  const float scale = a.scale;
  const float* gInit = a.init;
  float* gFinal = a.final_state;

  f32x4 S[SPW];
  const size_t st_off = ((size_t)seq * H + h) * DK * DV;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int ch = 16 * mt + 4 * q4 + ii, col = n0 + 16 * nt + r16;
      S[i][ii] = (gInit && t < NST) ? gInit[st_off + (size_t)ch * DV + col] : 0.f;
    }
  }

  // staging registers for the next chunk (separate objects so each stays in registers)
  TileCopy<E, CH, DK, NT> pw;
  TileCopy<E, (OUT ? CH : 1), (OUT ? DK : 16 / sizeof(E)), NT> pqt;
  TileCopy<float, DK, CH, NT> pkht;
  TileCopy<float, (OUT ? CH : 1), (OUT ? CH : 4), NT> paqk;
  TileCopy<float, DVS, CH, NT> put;
  TileCopy<float, 1, DK, NT> pgam;
  auto blk_of = [&](int n) { return (size_t)(c0 + n) * H + h; };
#define KDA_PRE_LOAD(n_)                                        \
  do {                                                          \
    const size_t b_ = blk_of(n_);                               \
    pw.load(gW + b_ * WB::W, DK);                               \
    if constexpr (OUT) {                                        \
      pqt.load(gQt + b_ * WB::QT, DK);                          \
      paqk.load(gAqk + b_ * WB::AQK, CH);                       \
    }                                                           \
    pkht.load(gKhT + b_ * WB::KHT, CH);                         \
    put.load(gUt + b_ * WB::UT + (size_t)n0 * CH, CH);          \
    pgam.load(gGam + b_ * WB::GAM, DK);                         \
  } while (0)
#define KDA_PRE_STORE()                                         \
  do {                                                          \
    pw.store(sW, L::LDK);                                       \
    if constexpr (OUT) {                                        \
      pqt.store(sQt, L::LDK);                                   \
      paqk.store(sAqk, L::LDF);                                 \
    }                                                           \
    pkht.store(sKhT, L::LDF);                                   \
    put.store(sUt, CH);                                         \
    pgam.store(sGam, DK);                                       \
  } while (0)

  if (nch > 0) {
    KDA_PRE_LOAD(0);
    KDA_PRE_STORE();
  }
  const size_t ro = (size_t)H * DV;
  for (int n = 0; n < nch; ++n) {
    // prefetch the next chunk into registers (the last chunk re-reads itself,
    // so the staging registers are defined on every path)
    KDA_PRE_LOAD(n + 1 < nch ? n + 1 : n);

    // S -> LDS as a split operand, transposed ([column][channel])
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        const int off = (16 * nt + r16) * L::LDK + 16 * mt + 4 * q4;
        store4_split<E>(sSTh + off, sSTl + off, S[i][0], S[i][1], S[i][2], S[i][3]);
        if constexpr (!OUT) {
          // backward needs the state entering every chunk: float [DV][DK] per chunk-head
          float* dst = gS + blk_of(n) * WB::S + (size_t)(n0 + 16 * nt + r16) * DK + 16 * mt + 4 * q4;
          *reinterpret_cast<f32x4*>(dst) = S[i];
        }
      }
    }
    __syncthreads();

    f32x4 o1[NTS];
    if (w < 4) {
      // X = W S (token tile w); U = U~ - X -> LDS as a split operand ([column][token])
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) {
        const f32x4 x = tile_mm_ps<E, DK>(sW, L::LDK, 16 * w, sSTh, sSTl, L::LDK, 16 * nt);
        const float* ut = sUt + (16 * nt + r16) * CH + 16 * w + 4 * q4;
        const int off = (16 * nt + r16) * L::LDT + 16 * w + 4 * q4;
        store4_split<E>(sULh + off, sULl + off, ut[0] - x[0], ut[1] - x[1], ut[2] - x[2], ut[3] - x[3]);
      }
    } else if constexpr (OUT) {
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) o1[nt] = tile_mm_ps<E, DK>(sQt, L::LDK, 16 * (w - 4), sSTh, sSTl, L::LDK, 16 * nt);
    }
    __syncthreads();

    if constexpr (OUT) {
      if (w >= 4) {
        const int tt = w - 4;
        const ChunkInfo ci = gChunks[c0 + n];
        O* oh = gOut + (size_t)ci.t0 * ro + (size_t)h * DV + n0;
#pragma unroll
        for (int nt = 0; nt < NTS; ++nt) {
          f32x4 x = o1[nt];
#pragma unroll
          for (int k = 0; k < CH; k += 32) {
            const SFrag<E> fa = sfrag_row<E>(sAqk, L::LDF, 16 * tt + r16, k + 8 * q4);
            const SFrag<E> fb = sfrag_pair<E>(sULh, sULl, L::LDT, 16 * nt + r16, k + 8 * q4);
            x = mma_ss(fa, fb, x);
          }
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int tok = 16 * tt + 4 * q4 + ii;
            if (tok < ci.len) oh[(size_t)tok * ro + 16 * nt + r16] = cvt<O>(scale * x[ii]);
          }
        }
      }
    }
    // S' = Gamma_C * S + Kh^T U
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        f32x4 x = zero4();
#pragma unroll
        for (int k = 0; k < CH; k += 32) {
          const SFrag<E> fa = sfrag_row<E>(sKhT, L::LDF, 16 * mt + r16, k + 8 * q4);
          const SFrag<E> fb = sfrag_pair<E>(sULh, sULl, L::LDT, 16 * nt + r16, k + 8 * q4);
          x = mma_ss(fa, fb, x);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) S[i][ii] = sGam[16 * mt + 4 * q4 + ii] * S[i][ii] + x[ii];
      }
    }
    __syncthreads();
    if (n + 1 < nch) KDA_PRE_STORE();
  }
#undef KDA_PRE_LOAD
#undef KDA_PRE_STORE

  if (gFinal) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int ch = 16 * mt + 4 * q4 + ii, col = n0 + 16 * nt + r16;
          gFinal[st_off + (size_t)ch * DV + col] = S[i][ii];
        }
      }
    }
  }
}

template <typename E, typename O, int DK, int DV, int DVS, bool OUT>
static hipError_t launch_state(const Args& a, hipStream_t st) {
  constexpr int NSL = DV / DVS;
  const int units = a.N * a.H;
  const int groups = (units + 7) / 8;
  const int grid = groups * 8 * NSL;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((kda_state<E, O, DK, DV, DVS, OUT>), dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

template <typename E, int DK, int DV, bool BWD>
static hipError_t launch_prep(const Args& a, hipStream_t st) {
  if (a.max_chunks == 0 || a.H == 0) return hipSuccess;
  hipLaunchKernelGGL((kda_prep<E, DK, DV, BWD>), dim3(a.max_chunks, a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename E, typename O, int DK, int DV>
hipError_t launch_fwd(const Args& a, hipStream_t st) {
  hipError_t e = launch_chunk_map(a, st);
  if (e != hipSuccess) return e;
  e = launch_prep<E, DK, DV, false>(a, st);
  if (e != hipSuccess) return e;
  return launch_state<E, O, DK, DV, 16, true>(a, st);
}

// front half of the backward pass: chunk map, chunk-local prep (also keeping
// T), and the states entering every chunk
template <typename E, int DK, int DV>
hipError_t launch_bwd_front(const Args& a, hipStream_t st) {
  hipError_t e = launch_chunk_map(a, st);
  if (e != hipSuccess) return e;
  e = launch_prep<E, DK, DV, true>(a, st);
  if (e != hipSuccess) return e;
  return launch_state<E, float, DK, DV, 16, false>(a, st);
}

#define KDA_INST(E, DK, DV)                                                                   \
  template hipError_t launch_fwd<E, float, DK, DV>(const Args&, hipStream_t);                 \
  template hipError_t launch_bwd_front<E, DK, DV>(const Args&, hipStream_t);
KDA_INST(bf16, 64, 64)
KDA_INST(bf16, 64, 128)
KDA_INST(bf16, 128, 64)
KDA_INST(bf16, 128, 128)
KDA_INST(float, 64, 64)
KDA_INST(float, 64, 128)
KDA_INST(float, 128, 64)
KDA_INST(float, 128, 128)
#undef KDA_INST
#define KDA_INST_BF16OUT(DK, DV) template hipError_t launch_fwd<bf16, bf16, DK, DV>(const Args&, hipStream_t);
KDA_INST_BF16OUT(64, 64)
KDA_INST_BF16OUT(64, 128)
KDA_INST_BF16OUT(128, 64)
KDA_INST_BF16OUT(128, 128)
#undef KDA_INST_BF16OUT

}  // namespace kda
